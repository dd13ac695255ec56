// moe_unpermute.hip -- gfx950 unpermute: the weighted topk reduction back to token order.
//
// What is computed: vLLM PR #14568, "permute/unpermute kernel for moe optimization",
// PR description (the expanded expert output is gathered back per token, scaled by
// topk_weight and summed over the topk slots).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_index() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveSize));
}

// ----------------------------------------------------------------------------
// Unpermute: one wave per (token, chunk of U*64 16-byte vectors).  The loads
// of all topk rows of the chunk are issued before any arithmetic (G rows at a
// time when topk is not a compile-time constant), then summed in fp32 in
// ascending k and rounded once to the element type.  A slot whose inverse
// index is -1 (its expert lives on another rank) is skipped: no load, no term;
// at topk >= 4 a token with no other slot gets a zero row stored by one wave.
// Any other index outside [0, N*topk) turns the token's row into NaN.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool kBF16, int U>
__device__ __forceinline__ void accumulate(float (&acc)[U][kBF16 ? 8 : 4], const u32x4 (&v)[U], float wk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (kBF16) {
                acc[u][2 * q] = __builtin_fmaf(wk, bf16_lo(v[u][q]), acc[u][2 * q]);
                acc[u][2 * q + 1] = __builtin_fmaf(wk, bf16_hi(v[u][q]), acc[u][2 * q + 1]);
            } else {
                acc[u][q] = __builtin_fmaf(wk, __uint_as_float(v[u][q]), acc[u][q]);
            }
        }
    }
}

// Unpermute kernels take separate __restrict__ pointers (not a struct) so the
// compiler can prove the index / weight reads are never clobbered by the
// output stores, which keeps those wave-uniform reads on the scalar path,
// off the in-order vector-memory counter that the row loads use.

// One work item of a compile-time topk: all topk indices and weights are
// read first (independent of each other), then every row load of the chunk
// is issued; `finish` weights, sums, rounds and stores.
template <bool kBF16, int K, int U>
struct UnpermuteItem {
    int32_t j[K];
    float wk[K];
    u32x4 v[K][U];
};

// Reads the token's topk indices and weights; true when every index is -1
// (no local slot: the token's row is zero).
template <bool kBF16, int K, int U>
__device__ __forceinline__ bool unpermute_indices(const float* __restrict__ wts, const int32_t* __restrict__ inv,
                                                  int64_t t, UnpermuteItem<kBF16, K, U>& it) {
    bool remote = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        it.j[k] = inv[t * K + k];
        it.wk[k] = wts[t * K + k];
        remote &= it.j[k] == -1;
    }
    return remote;
}

// Issues the row loads of the chunk for the indices read by unpermute_indices.
template <bool kBF16, int K, int U>
__device__ __forceinline__ void unpermute_issue(const u32x4* __restrict__ y, int64_t R, int64_t rv, int64_t base,
                                                UnpermuteItem<kBF16, K, U>& it) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool ok = it.j[k] >= 0 && (int64_t)it.j[k] < R;
        if (!ok) it.wk[k] = 0.0f;  // the zero row then adds exactly nothing
        const u32x4* src = y + (int64_t)(ok ? it.j[k] : 0) * rv;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWaveSize;
            it.v[k][u] = (ok && idx < rv) ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <bool kBF16, int U>
__device__ __forceinline__ void store_outputs(u32x4* __restrict__ out, int64_t rv, int64_t base,
                                              const float (&acc)[U][kBF16 ? 8 : 4], bool bad) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t idx = base + u * kWaveSize;
        if (idx >= rv) continue;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (kBF16) {
                o[q] = bad ? 0x7FC07FC0u : (bf16_bits(acc[u][2 * q]) | (bf16_bits(acc[u][2 * q + 1]) << 16));
            } else {
                o[q] = bad ? 0x7FC00000u : __float_as_uint(acc[u][q]);
            }
        }
        __builtin_nontemporal_store(o, out + idx);
    }
}

template <bool kBF16, int K, int U>
__device__ __forceinline__ void unpermute_finish(u32x4* __restrict__ out, int64_t R, int64_t rv, int64_t t,
                                                 int64_t base, const UnpermuteItem<kBF16, K, U>& it) {
    constexpr int kEl = kBF16 ? 8 : 4;
    float acc[U][kEl];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kEl; ++e) acc[u][e] = 0.0f;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        bad |= !(it.j[k] >= -1 && (int64_t)it.j[k] < R);
        accumulate<kBF16, U>(acc, it.v[k], it.wk[k]);
    }
    store_outputs<kBF16, U>(out + t * rv, rv, base, acc, bad);
}

// A token whose every slot is -1 has all its experts on other ranks: its
// output row is zero.  The wave of the row's first chunk stores the whole row
// and the waves of its other chunks have nothing to do.  A zero row takes no
// loads, so with one wave per 1 KiB chunk nearly all of a wave's time would go
// to the index read (measured at the DSv3 shape, one rank of an 8-way expert
// split: that rank's unpermute 101 -> 71 us).  Only for topk >= 4: with fewer
// slots a token is rarely remote in every one (about a fifth of the tokens of
// a 2-way split at topk 2), and the test itself cost the plain topk-2
// unpermute 0.3 us per call (Mixtral shape).  This is the test for a run-time
// topk; with a compile-time topk unpermute_indices makes it on the indices it
// reads anyway.
constexpr int kZeroRowMinTopk = 4;

__device__ __forceinline__ bool token_is_remote(const int32_t* __restrict__ inv, int64_t t, int K) {
    bool remote = true;
    for (int k = 0; k < K; ++k) remote &= inv[t * K + k] == -1;
    return remote;
}

// Zeros over a whole row of rv vectors (the bits of +0.0, as the weighted sum
// over no slot rounds to); row is the token's output row.
__device__ __forceinline__ void store_zero_row(u32x4* __restrict__ row, int64_t rv, int lane) {
    for (int64_t c = lane; c < rv; c += kWaveSize) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, row + c);
}

// Item -> (token, first vector of this lane).  The token is the same for the
// whole wave, which readfirstlane makes explicit.
__device__ __forceinline__ void item_position(int64_t item, int64_t nchunks, int chunk_vecs, int64_t& t,
                                              int64_t& base) {
    t = __builtin_amdgcn_readfirstlane((int)(item / nchunks));
    base = (item - t * nchunks) * chunk_vecs + (int)(threadIdx.x % kWaveSize);
}

// KC > 0: topk is exactly KC.  KC == 0: runtime topk, rows taken G at a time.
// One item (token, chunk of U*64 vectors) per wave; only when the grid would
// exceed kMaxGridBlocks does a wave loop over items g, g + total_waves, ...
template <bool kBF16, int KC, int U, int G>
__global__ __launch_bounds__(256) void unpermute_kernel(const u32x4* __restrict__ y, const float* __restrict__ wts,
                                                        const int32_t* __restrict__ inv, u32x4* __restrict__ out,
                                                        int64_t num_tokens, int64_t rv, int topk,
                                                        int64_t total_waves) {
    constexpr int kEl = kBF16 ? 8 : 4;  // elements per 16-byte vector
    constexpr int kGroup = KC > 0 ? KC : G;
    const int64_t nchunks = (rv + U * kWaveSize - 1) / (U * kWaveSize);
    const int64_t items = num_tokens * nchunks;
    const int K = KC > 0 ? KC : topk;
    const int64_t R = num_tokens * K;
    const int lane = (int)(threadIdx.x % kWaveSize);
    for (int64_t item = (int64_t)blockIdx.x * (256 / kWaveSize) + wave_index(); item < items; item += total_waves) {
        int64_t t, base;
        item_position(item, nchunks, U * kWaveSize, t, base);
        if constexpr (KC > 0) {
            UnpermuteItem<kBF16, KC, U> it;
            if (unpermute_indices<kBF16, KC, U>(wts, inv, t, it) && KC >= kZeroRowMinTopk) {
                if (base == lane) store_zero_row(out + t * rv, rv, lane);  // the token's first chunk
                continue;
            }
            unpermute_issue<kBF16, KC, U>(y, R, rv, base, it);
            unpermute_finish<kBF16, KC, U>(out, R, rv, t, base, it);
        } else {
            if (K >= kZeroRowMinTopk && token_is_remote(inv, t, K)) {
                if (base == lane) store_zero_row(out + t * rv, rv, lane);
                continue;
            }
            float acc[U][kEl];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < kEl; ++e) acc[u][e] = 0.0f;
            bool bad = false;
            for (int k0 = 0; k0 < K; k0 += kGroup) {
                int32_t j[kGroup];
                float wk[kGroup];
#pragma unroll
                for (int g = 0; g < kGroup; ++g) {
                    const bool live = k0 + g < K;
                    j[g] = live ? inv[t * K + k0 + g] : 0;
                    wk[g] = live ? wts[t * K + k0 + g] : 0.0f;
                }
                u32x4 v[kGroup][U];
#pragma unroll
                for (int g = 0; g < kGroup; ++g) {
                    const bool live = k0 + g < K;
                    const bool ok = live && j[g] >= 0 && (int64_t)j[g] < R;
                    bad |= live && !(j[g] >= -1 && (int64_t)j[g] < R);
                    if (!ok) wk[g] = 0.0f;
                    const u32x4* src = y + (int64_t)(ok ? j[g] : 0) * rv;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t idx = base + u * kWaveSize;
                        v[g][u] = (ok && idx < rv) ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
                    }
                }
#pragma unroll
                for (int g = 0; g < kGroup; ++g)
                    if (k0 + g < K) accumulate<kBF16, U>(acc, v[g], wk[g]);
            }
            store_outputs<kBF16, U>(out + t * rv, rv, base, acc, bad);
        }
    }
}

// ----------------------------------------------------------------------------
// Span schedule for the inverse index of an expert split (moe_unpermute_local,
// topk 8).  With one or two live slots per token, one wave per 1 KiB chunk
// keeps only 1-2 KiB of row loads in flight and the reduction is latency
// bound.  Here a wave owns a span of kSpanChunks chunks of one token, gathers
// the token's live slots (ascending k) and sums P chunks at a time, P chosen
// so that live slots x P is about eight row loads in flight: one slot takes
// all four chunks at once, two slots four, three or four slots two, five or
// more one.  The loads of the next P chunks are issued before the stores of
// the current ones (one counter covers both on this chip, in issue order, so
// waiting for loads issued after a store would wait for the store too).
// Terms are added in ascending k exactly as the per-chunk kernel adds them
// (a -1 slot there adds 0 * 0, which leaves a sum that started at +0 unchanged),
// so both schedules give the same bits.
// ----------------------------------------------------------------------------
constexpr int kSpanChunks = 4;
// Spans (tokens x spans per token) from which the span schedule is used: the
// DSv3 shape (16384 tokens x 4 spans) took one 8-way rank's unpermute
// 110 -> 95 us and the other ranks 69 -> 66 and 73 -> 69 us; the Qwen3 shape
// (8192 tokens x 1 span, 4-way split) ran slower with it (18 -> 21 us), too
// few waves for the machine.
constexpr int64_t kSpanMinItems = 32768;

template <int LC, int P>
__device__ __forceinline__ void span_load(const u32x4* __restrict__ y, int64_t rv, int64_t c0, int64_t c_end,
                                          const int32_t (&jc)[LC], int nlive, int lane, u32x4 (&v)[LC][P]) {
#pragma unroll
    for (int l = 0; l < LC; ++l) {
        const u32x4* src = y + (int64_t)jc[l] * rv;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t idx = (c0 + p) * kWaveSize + lane;
            const bool ok = l < nlive && c0 + p < c_end && idx < rv;
            v[l][p] = ok ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// The span [c_begin, c_end) of token row orow from the nlive compacted slots.
template <bool kBF16, int LC, int P>
__device__ __forceinline__ void span_sum(const u32x4* __restrict__ y, u32x4* __restrict__ orow, int64_t rv,
                                         int64_t c_begin, int64_t c_end, const int32_t (&jc)[LC],
                                         const float (&wc)[LC], int nlive, int lane) {
    constexpr int kEl = kBF16 ? 8 : 4;
    u32x4 v[LC][P];
    span_load<LC, P>(y, rv, c_begin, c_end, jc, nlive, lane, v);
    for (int64_t c0 = c_begin; c0 < c_end; c0 += P) {
        float acc[P][1][kEl];
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int e = 0; e < kEl; ++e) acc[p][0][e] = 0.0f;
#pragma unroll
        for (int l = 0; l < LC; ++l) {
            if (l < nlive) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const u32x4 one[1] = {v[l][p]};
                    accumulate<kBF16, 1>(acc[p], one, wc[l]);
                }
            }
        }
        if (c0 + P < c_end) span_load<LC, P>(y, rv, c0 + P, c_end, jc, nlive, lane, v);
#pragma unroll
        for (int p = 0; p < P; ++p)
            if (c0 + p < c_end) store_outputs<kBF16, 1>(orow, rv, (c0 + p) * kWaveSize + lane, acc[p], false);
    }
}

// Compacts the live slots (mask bit k: slot k live) into the first LC entries,
// ascending k, with selects only (a run-time index into the slot arrays would
// put them in scratch or LDS), then sums the span.
template <bool kBF16, int LC, int P>
__device__ __forceinline__ void span_compact(const u32x4* __restrict__ y, u32x4* __restrict__ orow, int64_t rv,
                                             int64_t c_begin, int64_t c_end, const int32_t (&j)[8],
                                             const float (&wk)[8], uint32_t mask, int lane) {
    int32_t jc[LC];
    float wc[LC];
#pragma unroll
    for (int l = 0; l < LC; ++l) {
        jc[l] = 0;
        wc[l] = 0.0f;
    }
    int n = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool live = (mask >> k) & 1u;
#pragma unroll
        for (int l = 0; l < LC; ++l) {
            const bool here = live && n == l;
            jc[l] = here ? j[k] : jc[l];
            wc[l] = here ? wk[k] : wc[l];
        }
        n += live ? 1 : 0;
    }
    span_sum<kBF16, LC, P>(y, orow, rv, c_begin, c_end, jc, wc, n < LC ? n : LC, lane);
}

template <bool kBF16>
__global__ __launch_bounds__(256) void unpermute_span_kernel(const u32x4* __restrict__ y,
                                                             const float* __restrict__ wts,
                                                             const int32_t* __restrict__ inv,
                                                             u32x4* __restrict__ out, int64_t num_tokens,
                                                             int64_t rv, int64_t total_waves) {
    constexpr int K = 8;
    constexpr int C = kSpanChunks;
    const int64_t nchunks = (rv + kWaveSize - 1) / kWaveSize;
    const int64_t nspans = (nchunks + C - 1) / C;
    const int64_t items = num_tokens * nspans;
    const int64_t R = num_tokens * K;
    const int lane = (int)(threadIdx.x % kWaveSize);
    for (int64_t item = (int64_t)blockIdx.x * (256 / kWaveSize) + wave_index(); item < items; item += total_waves) {
        const int64_t t = __builtin_amdgcn_readfirstlane((int)(item / nspans));
        const int64_t c_begin = (item - t * nspans) * C;
        const int64_t c_end = c_begin + C < nchunks ? c_begin + C : nchunks;
        int32_t j[K];
        float wk[K];
        uint32_t mask = 0;
        bool bad = false;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            j[k] = inv[t * K + k];
            wk[k] = wts[t * K + k];
            bad |= !(j[k] >= -1 && (int64_t)j[k] < R);
            mask |= (j[k] >= 0 ? 1u : 0u) << k;
        }
        u32x4* orow = out + t * rv;
        if (bad || mask == 0) {  // NaN row (bad index) or zero row (every slot remote)
            const uint32_t fill = bad ? (kBF16 ? 0x7FC07FC0u : 0x7FC00000u) : 0u;
            for (int64_t idx = c_begin * kWaveSize + lane; idx < c_end * kWaveSize && idx < rv; idx += kWaveSize)
                __builtin_nontemporal_store(u32x4{fill, fill, fill, fill}, orow + idx);
            continue;
        }
        const int live = __builtin_popcount(mask);
        if (live >= 5) span_compact<kBF16, 8, 1>(y, orow, rv, c_begin, c_end, j, wk, mask, lane);
        else if (live >= 3) span_compact<kBF16, 4, 2>(y, orow, rv, c_begin, c_end, j, wk, mask, lane);
        else if (live == 2) span_compact<kBF16, 2, C>(y, orow, rv, c_begin, c_end, j, wk, mask, lane);
        else span_compact<kBF16, 1, C>(y, orow, rv, c_begin, c_end, j, wk, mask, lane);
    }
}

// Occupancy cap for large topk-8 reductions whose slots are all live.  At the
// DSv3 shape (N = 16384, rows of 14 KiB, 57344 workgroups) three workgroups
// of four waves per CU measured 367 -> 350 us for the unpermute alone and
// 802 -> 765 us for the permute + unpermute step (the permute after it runs
// faster as well); two, four, five and six workgroups per CU were slower than
// three.  What helps is fewer resident waves, not fewer bytes in flight:
// waves that issue their eight row loads in groups of four or two (every CU
// slot filled) measured the same as all eight at once, 366-367 us, and so
// did waves that sum chunks of two tokens at once.  Small grids need every
// slot to cover memory latency (Qwen3 shape, 8192 workgroups: fastest
// uncapped), so the cap applies from kUnpermuteCapMinBlocks workgroups on.
// Inverse indices of an expert split (moe_unpermute_local) are not capped:
// with one or two live slots per token a wave is latency bound, and the cap
// made one rank's unpermute at the DSv3 shape, 8-way split, 110 -> 163 us.
// The cap is imposed through dynamic LDS that the kernel never touches: each
// workgroup reserves just over a quarter of the CU's LDS, so at most three
// fit on a CU.
constexpr int kUnpermuteCapTopk = 8;
constexpr int64_t kUnpermuteCapMinBlocks = 16384;
constexpr int kUnpermuteCapWorkgroups = 3;
constexpr int kMaxDevices = 64;

// LDS bytes per workgroup that let at most kUnpermuteCapWorkgroups workgroups
// share a CU of the current device; 0 when the device cannot be queried.
static size_t unpermute_cap_lds_bytes() {
    static std::atomic<int> lds_per_cu[kMaxDevices];  // 0: not queried yet, -1: query failed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = lds_per_cu[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            v <= 0)
            v = -1;
        lds_per_cu[dev].store(v, std::memory_order_relaxed);
    }
    if (v < 0) return 0;
    // cap * bytes <= v < (cap + 1) * bytes, whatever the allocation granularity
    // (below v / (cap * (cap + 1)) bytes)
    return (size_t)(v / (kUnpermuteCapWorkgroups + 1)) + 1;
}

template <bool kBF16>
static hipError_t launch_unpermute_span(const UnpermuteArgs& a, int64_t items, hipStream_t stream) {
    const int64_t blocks_needed = (items + 3) / 4;
    const int64_t blocks = blocks_needed < kMaxGridBlocks ? blocks_needed : kMaxGridBlocks;
    hipLaunchKernelGGL((unpermute_span_kernel<kBF16>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(a.expanded_output), a.topk_weights, a.inv_permuted_idx,
                       reinterpret_cast<u32x4*>(a.output), a.num_tokens, a.row_vecs, blocks * 4);
    return hipGetLastError();
}

template <bool kBF16, int KC, int U, int G>
static hipError_t launch_unpermute_t(const UnpermuteArgs& a, hipStream_t stream) {
    if (KC == 8 && a.few_live) {
        const int64_t spans = a.num_tokens * (((a.row_vecs + kWaveSize - 1) / kWaveSize + kSpanChunks - 1) / kSpanChunks);
        if (spans >= kSpanMinItems) return launch_unpermute_span<kBF16>(a, spans, stream);
    }
    const int64_t nchunks = (a.row_vecs + U * kWaveSize - 1) / (U * kWaveSize);
    const int64_t items = a.num_tokens * nchunks;
    const int64_t blocks_needed = (items + 3) / 4;
    const int64_t blocks = blocks_needed < kMaxGridBlocks ? blocks_needed : kMaxGridBlocks;
    const size_t lds = !a.few_live && KC == kUnpermuteCapTopk && blocks >= kUnpermuteCapMinBlocks
                           ? unpermute_cap_lds_bytes()
                           : 0;
    hipLaunchKernelGGL((unpermute_kernel<kBF16, KC, U, G>), dim3((unsigned)blocks), dim3(256), lds, stream,
                       reinterpret_cast<const u32x4*>(a.expanded_output), a.topk_weights, a.inv_permuted_idx,
                       reinterpret_cast<u32x4*>(a.output), a.num_tokens, a.row_vecs, a.topk, blocks * 4);
    return hipGetLastError();
}


// Unpermute dispatch: one item per wave, one 16-byte vector per lane (a
// chunk is 64 vectors = 1 KiB of each of the topk rows).  Measured on MI355X
// against 2, 4 and 7-8 vectors per lane and against persistent pipelined
// waves: the narrowest chunks, i.e. the most waves in flight, were fastest for
// every workload once the index reads stayed on the scalar path.
template <bool kBF16, int KC, int G>
static hipError_t launch_unpermute_k(const UnpermuteArgs& a, hipStream_t stream) {
    return launch_unpermute_t<kBF16, KC, 1, G>(a, stream);
}

template <bool kBF16>
static hipError_t launch_unpermute_dtype(const UnpermuteArgs& a, hipStream_t stream) {
    switch (a.topk) {
        case 1: return launch_unpermute_k<kBF16, 1, 1>(a, stream);
        case 2: return launch_unpermute_k<kBF16, 2, 2>(a, stream);
        case 4: return launch_unpermute_k<kBF16, 4, 4>(a, stream);
        case 8: return launch_unpermute_k<kBF16, 8, 8>(a, stream);
        default: return launch_unpermute_k<kBF16, 0, 4>(a, stream);
    }
}

hipError_t launch_unpermute(const UnpermuteArgs& a, bool bf16, hipStream_t stream) {
    return bf16 ? launch_unpermute_dtype<true>(a, stream) : launch_unpermute_dtype<false>(a, stream);
}

}  // namespace moe
