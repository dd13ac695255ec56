// moe_permute_coarse.hip -- coarse permute schedule (two kernels: coarse histogram, then scatter).
// What is computed and how ranks stay stable: see moe_permute_device.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

// ----------------------------------------------------------------------------
// Coarse permute, kernel 1 of 2: bucket counts of each coarse tile of
// coarse_rows expanded rows.  hist[c][b] = rows of coarse tile c with key b;
// hist[c][B] = rows with a bad id or map entry.  Rows of remote experts are
// not counted.
// ----------------------------------------------------------------------------
template <int NT, bool kMap, typename IdT>
__global__ __launch_bounds__(NT) void permute_coarse_hist_kernel(const IdT* __restrict__ ids,
                                                                 const int32_t* __restrict__ expert_map, int R, int E,
                                                                 int B, int coarse_rows, int32_t* __restrict__ hist) {
    extern __shared__ int smem[];  // [B + 1], then the map [E] when there is one
    // Ids go out kBatch per thread at a time; the first batch before the LDS
    // set-up, so its loads overlap it (one load, wait and atomic after another
    // left the kernel a chain of memory round trips).
    constexpr int kBatch = 8;
    const int r0 = (int)blockIdx.x * coarse_rows;
    const int r1 = min(r0 + coarse_rows, R);
    int v[kBatch];
    auto load_batch = [&](int base) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int r = base + (int)threadIdx.x + q * NT;
            v[q] = r < r1 ? load_id(ids, r) : 0;
        }
    };
    load_batch(r0);
    int* map_w = smem + B + 1;
    for (int e = threadIdx.x; e <= B; e += NT) smem[e] = 0;
    if constexpr (kMap)
        for (int e = threadIdx.x; e < E; e += NT) map_w[e] = expert_map[e];
    lds_barrier();
    const int* map_s = map_w;
    for (int base = r0; base < r1; base += kBatch * NT) {
        if (base != r0) load_batch(base);
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int r = base + (int)threadIdx.x + q * NT;
            if (r < r1) {
                const int key = bucket_of<kMap>(v[q], E, map_s, B);
                if (key != kRemoteKey) atomicAdd(&smem[key >= 0 ? key : B], 1);
            }
        }
    }
    lds_barrier();
    int32_t* row = hist + (int64_t)blockIdx.x * (B + 1);
    for (int e = threadIdx.x; e <= B; e += NT) row[e] = smem[e];
}

// ----------------------------------------------------------------------------
// Coarse permute, kernel 2 of 2: one workgroup per tile of whole tokens, like
// the fused kernel, except that the counts outside the tile come from the
// coarse histogram (held in LDS) plus a count of the rows that precede the
// tile inside its own coarse tile.  Tiles never straddle coarse tiles.
// ----------------------------------------------------------------------------
// kHist / kPartial: batches of NT histogram entries / preceding ids each
// thread loads, chosen by the launcher (as for the fused kernel's ids: no
// load for entries that do not exist, no branch among the loads, and fewer
// registers held through the index phase).
template <int NT, int U, bool kNTStore, bool kMap, typename IdT, int kHist, int kPartial>
__global__ __launch_bounds__(NT) void permute_coarse_scatter_kernel(PermuteArgs a, int tokens_per_tile, int nbits,
                                                                    int coarse_rows, int num_coarse,
                                                                    const int32_t* __restrict__ hist) {
    constexpr int W = NT / kWaveSize;
    static_assert(kHist * NT <= kCoarseMaxHist && kPartial * NT <= kCoarseMaxRowsPerTile, "coarse load batches");
    constexpr int kBatches = (kMaxTileRows + NT - 1) / NT;
    constexpr int kPer = (kMaxExperts + NT - 1) / NT;
    static_assert(kCoarseMaxHist % NT == 0 && kCoarseMaxRowsPerTile % NT == 0, "coarse bounds vs workgroup size");
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int B = a.num_buckets;
    const int K = a.topk;
    const int w = wave_index();
    const int lane = threadIdx.x % kWaveSize;
    const int64_t t0 = (int64_t)blockIdx.x * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int row0 = (int)(t0 * K);
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;
    const int span = (T + NT - 1) / NT * kWaveSize;
    const int cc = row0 / coarse_rows;  // this tile's coarse tile
    const int c_start = cc * coarse_rows;
    const int hist_n = num_coarse * (B + 1);
    const IdT* ids = static_cast<const IdT*>(a.topk_ids);

    // Independent loads first: the coarse histogram, the rows that precede
    // this tile in its coarse tile, the map, this wave's tile keys; then row
    // chunks.
    int hv[kHist];
#pragma unroll
    for (int j = 0; j < kHist; ++j) {
        const int i = (int)threadIdx.x + j * NT;
        hv[j] = hist[i < hist_n ? i : hist_n - 1];
    }
    int pv[kPartial];
#pragma unroll
    for (int j = 0; j < kPartial; ++j) {
        const int r = c_start + (int)threadIdx.x + j * NT;
        pv[j] = load_id(ids, r < row0 ? r : row0);  // row0 is a valid row (T >= 1)
    }
    MapStage<NT, kMap> ms;
    ms.load(a);
    int tkey[kBatches];
    load_tile_keys<kBatches>(ids, row0, T, span, w, lane, tkey);
    const TileCopy<U, kNTStore, kMap, IdT> tc(a, t0, ntok);
    u32x4 cur[U];
    tc.prefetch(w, cur);

    int* hist_s = smem;                   // [num_coarse * (B + 1)]
    int* before_s = hist_s + hist_n;      // [B] preceding rows in the coarse tile, then the tile's base
    int* wave_s = before_s + B;           // [W * B]
    int* dest_s = wave_s + W * B;         // [tile_cap]
    int* misc_s = dest_s + tile_cap;      // [16]: [0] bad ids, [1..W] scan scratch
    const int* map_s = ms.store(a, misc_s + 16);  // [E] with a map

#pragma unroll
    for (int j = 0; j < kHist; ++j) {
        if (j * NT >= hist_n) break;  // the same for the whole workgroup
        const int i = (int)threadIdx.x + j * NT;
        if (i < hist_n) hist_s[i] = hv[j];
    }
    for (int i = threadIdx.x; i < (1 + W) * B; i += NT) before_s[i] = 0;
    if (threadIdx.x < 16) misc_s[threadIdx.x] = 0;
    lds_barrier();

    // Phase 1: preceding rows of the coarse tile (LDS atomics), ranks inside
    // each wave's span, and the bad-id total from the histogram.
#pragma unroll
    for (int j = 0; j < kPartial; ++j) {
        if (c_start + j * NT >= row0) break;  // the same for the whole workgroup
        const int r = c_start + (int)threadIdx.x + j * NT;
        if (r < row0) {
            if constexpr (kMap) {
                const int key = bucket_of<true>(pv[j], E, map_s, B);
                if (key >= 0) atomicAdd(&before_s[key], 1);
            } else {
                if ((unsigned)pv[j] < (unsigned)E) atomicAdd(&before_s[pv[j]], 1);
            }
        }
    }
    if constexpr (kMap) tile_keys_to_buckets<true, kBatches>(tkey, E, map_s, B);
    int trank[kBatches];
    rank_own_rows<kMap, kBatches>(tkey, T, span, E, nbits, w, lane, wave_s + w * B, trank);
    if (threadIdx.x == 0) {
        int bad = 0;
        for (int c = 0; c < num_coarse; ++c) bad += hist_s[c * (B + 1) + B];
        misc_s[0] = bad;
    }
    lds_barrier();
    if (misc_s[0] != 0) {  // the histogram covers every id, so all workgroups agree
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e <= B; e += NT) a.expert_first_token_offset[e] = -1;
        return;
    }

    // Phase 2: offsets and this tile's base per bucket.
    expert_bases<NT, kPer>(
        B, wave_s, before_s, misc_s + 1, a.expert_first_token_offset, blockIdx.x == 0,
        [&](int e, int) {
            int t = 0;
            for (int c = 0; c < num_coarse; ++c) t += hist_s[c * (B + 1) + e];
            return t;
        },
        [&](int e) {
            int b = before_s[e];
            for (int c = 0; c < cc; ++c) b += hist_s[c * (B + 1) + e];
            return b;
        });
    lds_barrier();

    // Phase 3: destinations, then the row copy.
    write_dests<kMap, kBatches>(a, tkey, trank, row0, T, span, B, w, lane, before_s, wave_s, dest_s);
    lds_barrier();
    if (a.row_vecs > 0) copy_items_pipelined<U, NT, kNTStore, kMap, IdT>(tc, cur, dest_s);
    copy_tile_scales<NT>(a, t0, ntok, dest_s);
}

template <int U, bool kMap, typename IdT, int kHist, int kPartial>
static void launch_coarse_hp(const PermuteArgs& a, const PermutePlan& p, const int32_t* hist, size_t lds,
                             hipStream_t stream) {
    if constexpr (U <= kPlainStoreMaxUnroll) {
        if (plain_row_stores(a)) {
            hipLaunchKernelGGL((permute_coarse_scatter_kernel<kCoarseThreads, U, false, kMap, IdT, kHist, kPartial>),
                               dim3((unsigned)p.num_tiles), dim3(kCoarseThreads), lds, stream, a, p.tokens_per_tile,
                               p.nbits, p.coarse_rows, p.num_coarse, hist);
            return;
        }
    }
    hipLaunchKernelGGL((permute_coarse_scatter_kernel<kCoarseThreads, U, true, kMap, IdT, kHist, kPartial>),
                       dim3((unsigned)p.num_tiles), dim3(kCoarseThreads), lds, stream, a, p.tokens_per_tile, p.nbits,
                       p.coarse_rows, p.num_coarse, hist);
}

// Coarse load batches per thread: 4 when the histogram (num_coarse * (B + 1)
// entries) or the rows before a tile in its coarse tile fit in 4 * 512, else
// 16 (DSv3-shaped 8-way expert split, lightly loaded rank: permute
// 64.0 -> 61.1 us with 4 histogram batches).
template <int U, bool kMap, typename IdT>
static void launch_coarse_v(const PermuteArgs& a, const PermutePlan& p, const int32_t* hist, hipStream_t stream) {
    const size_t lds = coarse_scatter_lds_bytes(a.num_buckets, p.tile_rows, p.num_coarse, map_entries(a));
    constexpr int kFew = 4, kMany = kCoarseMaxHist / kCoarseThreads;
    static_assert(kCoarseMaxRowsPerTile / kCoarseThreads == kMany, "one bound for both load batches");
    const bool few_hist = (int64_t)p.num_coarse * (a.num_buckets + 1) <= kFew * kCoarseThreads;
    const bool few_rows = (int64_t)p.coarse_rows - p.tile_rows <= kFew * kCoarseThreads;
    if (few_hist && few_rows) launch_coarse_hp<U, kMap, IdT, kFew, kFew>(a, p, hist, lds, stream);
    else if (few_hist) launch_coarse_hp<U, kMap, IdT, kFew, kMany>(a, p, hist, lds, stream);
    else if (few_rows) launch_coarse_hp<U, kMap, IdT, kMany, kFew>(a, p, hist, lds, stream);
    else launch_coarse_hp<U, kMap, IdT, kMany, kMany>(a, p, hist, lds, stream);
}

template <int U>
static void launch_coarse_u(const PermuteArgs& a, const PermutePlan& p, const int32_t* hist, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_coarse_v<U, kMap, IdT>(a, p, hist, stream);
    });
}

hipError_t launch_permute_coarse(const PermuteArgs& a, const PermutePlan& p, void* workspace, int u,
                                 hipStream_t stream) {
    const int B = a.num_buckets;
    const int M = map_entries(a);
    int32_t* hist = static_cast<int32_t*>(workspace);
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        hipLaunchKernelGGL((permute_coarse_hist_kernel<kCoarseThreads, kMap, IdT>), dim3((unsigned)p.num_coarse),
                           dim3(kCoarseThreads), coarse_hist_lds_bytes(B, M), stream,
                           static_cast<const IdT*>(a.topk_ids), a.expert_map, (int)p.rows, a.num_experts, B,
                           p.coarse_rows, hist);
    });
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
#define MOE_COARSE(U) launch_coarse_u<U>(a, p, hist, stream)
    MOE_DISPATCH_U(u, MOE_COARSE)
#undef MOE_COARSE
    return hipGetLastError();
}

}  // namespace moe
