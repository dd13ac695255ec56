// moe_permute_wave.hip -- permute schedule for small problems (decode): one
// wave per workgroup, no workgroup barrier.
//
// What is computed is moe_permute's (vLLM PR #14568, PR description: count the
// rows of each expert, scan the counts into expert_first_token_offset, order
// the expanded rows stably by expert, copy each token row to its topk
// destinations).  At decode sizes (N*topk <= kWaveMaxRows) the cost is the
// chain of dependent steps, not bytes: the fused schedule's 512-thread
// workgroups need five workgroup barriers between its phases.  Here every
// workgroup is a single wave that holds all expert ids (at most 2 per lane)
// and computes the whole index itself:
//   * stable ranks: the rows are walked in batches of 64 in ascending order;
//     inside a batch the lanes with the same expert are found with one ballot
//     per id bit and a row's rank is the count of such lanes below it (mbcnt)
//     plus the rows of its expert in earlier batches (a running count in LDS,
//     advanced by the lowest lane of each equal-key group);
//   * the running counts end as the rows per expert; their exclusive scan
//     (wave shuffles) gives the offsets, and destination = offset + rank.
// LDS operations of one wave complete in order, so the wave needs no barrier.
// Workgroups redundantly compute the index (at most 128 ids each,
// wave_index_pass in moe_permute_device.h) and each copies its own row chunks
// of one token (grid: chunks x tokens); workgroup (0, 0) writes the index
// outputs.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

// kPer: expert ids each lane holds (N*topk <= 64*kPer), chosen by the launcher.
// kScale: per-token scales move with the rows (loaded with the ids, so the
// writer's scale stores wait on no load of their own).
// kRows: rows are copied (row_vecs > 0); the grid then has at most one
// workgroup per row chunk of each token, so the first chunk's loads are
// unconditional (a branch among the loads would leave the compiler a run-time
// count of loads in flight, and it would wait for the row loads before
// consuming the ids).
template <bool kNTStore, typename IdT, int kPer, bool kRows, bool kScale>
__global__ __launch_bounds__(kWaveSize) void permute_wave_kernel(PermuteArgs a, int nbits) {
    constexpr int U = 1;  // one 16-byte vector per lane: the most waves for the few rows
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int K = a.topk;
    const int R = (int)(a.num_tokens * K);  // 1 <= R <= 64 * kPer
    int* run = smem;                        // [E] rows per expert so far, then the offsets
    int* dest_s = run + E;                  // [R] destination of each expanded row
    const int lane = (int)threadIdx.x;
    const IdT* ids = static_cast<const IdT*>(a.topk_ids);
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;

    // Independent loads first: every id, then this wave's first row chunk.
    int id[kPer];
    float sc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int r = j * kWaveSize + lane;
        id[j] = load_id(ids, r < R ? r : R - 1);
    }
    if constexpr (kScale) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int r = j * kWaveSize + lane;
            sc[j] = a.token_scale[(r < R ? r : R - 1) / K];
        }
    }
    // Workgroup (x, y) copies chunks x, x + gridDim.x, ... of token y's row
    // (a 2-D grid: no division on the way to the first load).  Lanes past the
    // row's end load its last vector and store nothing, so the loads are
    // unconditional.
    const int64_t rv = a.row_vecs;
    const int t = (int)blockIdx.y;
    const u32x4* src = static_cast<const u32x4*>(a.hidden_states) + (int64_t)t * rv;
    u32x4* dst = static_cast<u32x4*>(a.permuted_hidden_states);
    u32x4 v[U];
    auto load_chunk = [&](int64_t c) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = c * (U * kWaveSize) + u * kWaveSize + lane;
            v[u] = __builtin_nontemporal_load(src + (idx < rv ? idx : rv - 1));
        }
    };
    int64_t chunk = blockIdx.x;  // < the row's chunk count when kRows (the grid never exceeds it)
    if constexpr (kRows) load_chunk(chunk);

    if (!wave_index_pass<kPer, kScale>(E, R, nbits, id, sc, run, dest_s, writer, a.expert_first_token_offset,
                                       a.permuted_idx, a.inv_permuted_idx, a.permuted_scale))
        return;  // a rejected id: every workgroup saw it and stops here

    // Row copy of token t: chunk `chunk`, then chunk + gridDim.x, ...; the
    // next chunk's loads are issued before the current one is stored.
    if constexpr (kRows) {
        const int64_t nchunks = (rv + U * kWaveSize - 1) / (U * kWaveSize);
        for (; chunk < nchunks; chunk += gridDim.x) {
            u32x4 cur[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = v[u];
            if (chunk + gridDim.x < nchunks) load_chunk(chunk + gridDim.x);
            for (int k = 0; k < K; ++k) {
                u32x4* o = dst + (int64_t)dest_s[t * K + k] * rv;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t idx = chunk * (U * kWaveSize) + u * kWaveSize + lane;
                    if (idx < rv) {
                        if constexpr (kNTStore)
                            __builtin_nontemporal_store(cur[u], o + idx);
                        else
                            o[idx] = cur[u];
                    }
                }
            }
        }
    }
}

template <typename IdT, int kPer>
static void launch_wave_p(const PermuteArgs& a, const PermutePlan& p, hipStream_t stream) {
    const size_t lds = wave_lds_bytes(a.num_experts, (int)p.rows);
    if (a.row_vecs == 0) {  // indices only (the scales still move when given)
        if (a.token_scale != nullptr)
            hipLaunchKernelGGL((permute_wave_kernel<true, IdT, kPer, false, true>), dim3(1), dim3(kWaveSize), lds,
                               stream, a, p.nbits);
        else
            hipLaunchKernelGGL((permute_wave_kernel<true, IdT, kPer, false, false>), dim3(1), dim3(kWaveSize), lds,
                               stream, a, p.nbits);
        return;
    }
    const int64_t nchunks = (a.row_vecs + kWaveSize - 1) / kWaveSize;
    const dim3 grid((unsigned)(nchunks < kWaveMaxChunkBlocks ? nchunks : kWaveMaxChunkBlocks),
                    (unsigned)a.num_tokens);
    const bool nt = !plain_row_stores(a);
#define MOE_WAVE_LAUNCH(NT, SC)                                                                                     \
    hipLaunchKernelGGL((permute_wave_kernel<NT, IdT, kPer, true, SC>), grid, dim3(kWaveSize), lds, stream, a, \
                       p.nbits)
    if (a.token_scale != nullptr) {
        if (nt) MOE_WAVE_LAUNCH(true, true);
        else MOE_WAVE_LAUNCH(false, true);
    } else {
        if (nt) MOE_WAVE_LAUNCH(true, false);
        else MOE_WAVE_LAUNCH(false, false);
    }
#undef MOE_WAVE_LAUNCH
}

// Up to kWaveMaxRows = 128 rows: one or two ids per lane.  Measured against the
// fused schedule (decode, topk 8, graph replay): 8 rows 3.3 vs 4.8 us, 32 rows
// 3.3 vs 4.9, 128 rows 4.1 vs 5.1; 256 rows 5.3 vs 5.2 and 512 rows 8.2 vs 5.4,
// where the serial walk over the id batches in every wave outweighs the
// fused kernel's barriers.
template <typename IdT>
static void launch_wave_i(const PermuteArgs& a, const PermutePlan& p, hipStream_t stream) {
    static_assert(kWaveMaxRows == 2 * kWaveSize, "id registers per lane cover the wave schedule's rows");
    if (p.rows <= kWaveSize) launch_wave_p<IdT, 1>(a, p, stream);
    else launch_wave_p<IdT, 2>(a, p, stream);
}

// The row copy moves one 16-byte vector per lane per chunk whatever `u` the
// other schedules would take.
hipError_t launch_permute_wave(const PermuteArgs& a, const PermutePlan& p, int, hipStream_t stream) {
    if (a.ids64) launch_wave_i<int64_t>(a, p, stream);
    else launch_wave_i<int32_t>(a, p, stream);
    return hipGetLastError();
}

}  // namespace moe
