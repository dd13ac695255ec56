// moe_permute_rows.hip -- row copy of the split permute schedule: the index is
// written first (by the index-only schedules), then this kernel moves the rows.
//
// What is computed is moe_permute's copy step (vLLM PR #14568, PR
// description: each token row goes to its topk destinations in expert
// order): permuted_hidden_states[inv_permuted_idx[t*topk + k]] = hidden[t].
//
// For the largest copies (more than a GiB of expanded rows) this is faster
// than copying inside the index kernels: every wave owns one chunk of one
// token row and nothing else, so there is no index work, workgroup barrier or
// LDS traffic between its loads and its stores, and the wave count is large
// enough to keep every CU streaming.  Measured at the DSv3 shape (N = 16384,
// rows of 14 KiB, topk 8; 1.88 GB written): index pass 11 us + this copy
// 405 us against 434 us for the coarse schedule's copying kernels.
//
// The index pass sets every offset to -1 and writes no index when it meets an
// invalid expert id; the copy then reads expert_first_token_offset[0] (0 after
// a valid index pass) and writes nothing.  Every destination is checked
// against [0, N*topk) as well.  With an expert map (kMap) a row of another
// rank has destination -1 and is skipped, and a token with no local row is
// not read: its wave reads the destinations first.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

// One wave per (token, chunk of U*64 vectors).  KC > 0: topk is exactly KC;
// KC == 0: runtime topk.  The chunk's loads are issued first and
// unconditionally (lanes past the row end reload its last vector and store
// nothing), then the wave-uniform destinations are read; the loads are in
// bounds whatever the index pass found, so the check of its result waits
// until they are in flight.
template <int U, bool kNTStore, int KC, bool kMap>
__global__ __launch_bounds__(256) void permute_rows_kernel(const u32x4* __restrict__ x,
                                                           const int32_t* __restrict__ inv,
                                                           const int64_t* __restrict__ off,
                                                           u32x4* __restrict__ xp, int64_t num_tokens, int64_t rv,
                                                           int topk, int64_t total_waves) {
    const int K = KC > 0 ? KC : topk;
    const int64_t rows = num_tokens * K;
    const int64_t nchunks = (rv + U * kWaveSize - 1) / (U * kWaveSize);
    const int64_t items = num_tokens * nchunks;
    const int lane = (int)(threadIdx.x % kWaveSize);
    for (int64_t item = (int64_t)blockIdx.x * (256 / kWaveSize) + wave_index(); item < items; item += total_waves) {
        const int64_t t = __builtin_amdgcn_readfirstlane((int)(item / nchunks));
        const int64_t base = (item - t * nchunks) * (U * kWaveSize) + lane;
        const u32x4* src = x + t * rv;
        if constexpr (kMap) {
            // tokens with no local row are not read
            bool any = false;
            for (int k = 0; k < K; ++k) any |= inv[t * K + k] >= 0;
            if (!any) continue;
        }
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWaveSize;
            v[u] = __builtin_nontemporal_load(src + (idx < rv ? idx : rv - 1));
        }
        // off[0] != 0: the index pass rejected an expert id and every store
        // is skipped.  It is read after the row loads, as a vector load (an
        // index the compiler cannot see through keeps it from being hoisted),
        // so waiting for it coincides with waiting for the rows, where a
        // scalar read first would hold back the row loads by its latency.
        __builtin_amdgcn_sched_barrier(0);
        int64_t zero = 0;
        asm volatile("" : "+v"(zero));
        const int64_t live_rows = __builtin_amdgcn_readfirstlane((int)(off[zero] != 0)) ? 0 : rows;
        auto put = [&](int32_t d) {
            if ((uint64_t)(int64_t)d >= (uint64_t)live_rows) return;
            u32x4* dst = xp + (int64_t)d * rv;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = base + u * kWaveSize;
                if (idx < rv) {
                    if constexpr (kNTStore)
                        __builtin_nontemporal_store(v[u], dst + idx);
                    else
                        dst[idx] = v[u];
                }
            }
        };
        if constexpr (KC > 0) {
            int32_t d[KC];
#pragma unroll
            for (int k = 0; k < KC; ++k) d[k] = inv[t * KC + k];
#pragma unroll
            for (int k = 0; k < KC; ++k) put(d[k]);
        } else {
            for (int k = 0; k < K; ++k) put(inv[t * K + k]);
        }
    }
}

// Four vectors per lane (a 4 KiB chunk): measured at the DSv3 shape against
// one, two, three, six and eight (413-425 us for the others, 405 us here).
// With an expert map two (2 KiB chunks): one rank of an 8-way DSv3 split,
// ranks 0, 3 and 7: 116.0 -> 113.9, 46.4 -> 45.1 and 51.7 -> 49.5 us against
// four (one: 107.3, 59.4 and 61.8 us; eight: 117.5, 47.7 and 53.2 us).
constexpr int kRowsCopyUnroll = 4;
constexpr int kRowsCopyUnrollMap = 2;

template <bool kNT, int KC, bool kMap>
static void launch_rows_k(const PermuteArgs& a, hipStream_t stream) {
    constexpr int U = kMap ? kRowsCopyUnrollMap : kRowsCopyUnroll;
    const int64_t nchunks = (a.row_vecs + U * kWaveSize - 1) / (U * kWaveSize);
    const int64_t items = a.num_tokens * nchunks;
    const int64_t needed = (items + 3) / 4;
    const int64_t blocks = needed < kMaxGridBlocks ? needed : kMaxGridBlocks;
    hipLaunchKernelGGL((permute_rows_kernel<U, kNT, KC, kMap>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(a.hidden_states), a.inv_permuted_idx, a.expert_first_token_offset,
                       static_cast<u32x4*>(a.permuted_hidden_states), a.num_tokens, a.row_vecs, a.topk, blocks * 4);
}

template <bool kNT, bool kMap>
static void launch_rows_nt(const PermuteArgs& a, hipStream_t stream) {
    switch (a.topk) {
        case 8: launch_rows_k<kNT, 8, kMap>(a, stream); break;
        case 4: launch_rows_k<kNT, 4, kMap>(a, stream); break;
        case 2: launch_rows_k<kNT, 2, kMap>(a, stream); break;
        default: launch_rows_k<kNT, 0, kMap>(a, stream); break;
    }
}

hipError_t launch_permute_rows(const PermuteArgs& a, hipStream_t stream) {
    const bool m = a.expert_map != nullptr;
    if (plain_row_stores(a)) { if (m) launch_rows_nt<false, true>(a, stream); else launch_rows_nt<false, false>(a, stream); }
    else { if (m) launch_rows_nt<true, true>(a, stream); else launch_rows_nt<true, false>(a, stream); }
    return hipGetLastError();
}

}  // namespace moe
