// moe_permute_fused.hip -- fused permute schedule (one kernel; N*topk <= 16384 rows).
// What is computed and how ranks stay stable: see moe_permute_device.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

// ----------------------------------------------------------------------------
// Fused permute: one workgroup per tile of whole tokens.  Every workgroup
// counts the expert ids of all rows outside its tile (before / after it),
// ranks its own rows, derives expert_first_token_offset and its own base per
// expert, scatters permuted_idx / inv_permuted_idx and copies its rows.
// ----------------------------------------------------------------------------
// kIds: expert ids each thread holds (kIds * NT >= N * topk), a compile-time
// choice of the launcher, so no id load is issued for rows that do not exist
// and no branch sits among the loads (a branch there leaves the compiler a
// run-time count of loads in flight, and it then waits for all of them,
// the row prefetch included, before the ids are used).
template <int NT, int U, bool kNTStore, bool kMap, typename IdT, int kIds>
__global__ __launch_bounds__(NT) void permute_fused_kernel(PermuteArgs a, int tokens_per_tile, int nbits) {
    constexpr int W = NT / kWaveSize;
    static_assert(kIds * NT <= kFusedMaxRows, "id batches per thread cover at most the fused row bound");
    constexpr int kBatches = (kMaxTileRows + NT - 1) / NT;         // tile batches of 64 per wave
    constexpr int kPer = (kMaxExperts + NT - 1) / NT;              // buckets per thread in the scan
    static_assert(kFusedMaxRows % NT == 0, "fused row bound must be a multiple of the workgroup size");
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
    const int R = (int)(a.num_tokens * K);  // <= kFusedMaxRows
    const int span = (T + NT - 1) / NT * kWaveSize;
    const IdT* ids = static_cast<const IdT*>(a.topk_ids);

    // Loads, all independent: every expert id of the problem, the map, this
    // wave's own tile rows, then the first row chunk of this wave.  The
    // vector-memory counter retires in issue order, so the row loads stay in
    // flight while the ids are consumed.
    int idv[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int r = (int)threadIdx.x + j * NT;
        if constexpr (sizeof(IdT) == 8) {  // skip batches wholly past R: 8-byte ids cost twice the L2 reads
            idv[j] = 0;
            if (j * NT < R) idv[j] = load_id(ids, r < R ? r : R - 1);
        } else {  // int32: unconditional loads measured faster, even when most are repeats
            idv[j] = load_id(ids, r < R ? r : R - 1);
        }
    }
    MapStage<NT, kMap> ms;
    ms.load(a);
    int tkey[kBatches];
    load_tile_keys<kBatches>(ids, row0, T, span, w, lane, tkey);
    const TileCopy<U, kNTStore, kMap, IdT> tc(a, t0, ntok);
    u32x4 cur[U];
    tc.prefetch(w, cur);

    int* before_s = smem;                 // [B] rows before the tile, then the tile's base per bucket
    int* after_s = before_s + B;          // [B] rows after the tile
    int* wave_s = after_s + B;            // [W * B] per-wave counts inside the tile, then prefixes
    int* dest_s = wave_s + W * B;         // [tile_cap] destination of each tile row
    int* misc_s = dest_s + tile_cap;      // [16]: [0] bad ids, [1..W] scan scratch
    const int* map_s = ms.store(a, misc_s + 16);  // [E] with a map

    for (int i = threadIdx.x; i < (2 + W) * B; i += NT) smem[i] = 0;
    if (threadIdx.x < 16) misc_s[threadIdx.x] = 0;
    lds_barrier();

    // Phase 1: counts outside the tile (LDS atomics, order-free) and stable
    // ranks inside each wave's span of the tile.
    int nbad = 0;
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        if (j * NT >= R) break;  // the same for the whole workgroup; matters at decode sizes
        const int r = (int)threadIdx.x + j * NT;
        if (r < R && (r < row0 || r >= row0 + T)) {
            if constexpr (kMap) {
                const int key = bucket_of<true>(idv[j], E, map_s, B);
                nbad += key == kBadKey ? 1 : 0;
                if (key >= 0) atomicAdd(r < row0 ? &before_s[key] : &after_s[key], 1);
            } else {
                const int key = idv[j];
                const bool ok = (unsigned)key < (unsigned)E;
                nbad += ok ? 0 : 1;
                if (ok) atomicAdd(r < row0 ? &before_s[key] : &after_s[key], 1);
            }
        }
    }
    if constexpr (kMap) tile_keys_to_buckets<true, kBatches>(tkey, E, map_s, B);
    int trank[kBatches];
    nbad += rank_own_rows<kMap, kBatches>(tkey, T, span, E, nbits, w, lane, wave_s + w * B, trank);
    if (nbad) atomicAdd(&misc_s[0], nbad);
    lds_barrier();
    if (misc_s[0] != 0) {  // every workgroup saw every id, so all take this branch together
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e <= B; e += NT) a.expert_first_token_offset[e] = -1;
        return;
    }

    // Phase 2: offsets and this tile's base per bucket.
    expert_bases<NT, kPer>(
        B, wave_s, before_s, misc_s + 1, a.expert_first_token_offset, blockIdx.x == 0,
        [&](int e, int in_tile) { return before_s[e] + in_tile + after_s[e]; }, [&](int e) { return before_s[e]; });
    lds_barrier();

    // Phase 3: destinations of this wave's tile rows, then the row copy.
    write_dests<kMap, kBatches>(a, tkey, trank, row0, T, span, B, w, lane, before_s, wave_s, dest_s);
    lds_barrier();
    if (a.row_vecs > 0) copy_items_pipelined<U, NT, kNTStore, kMap, IdT>(tc, cur, dest_s);
    copy_tile_scales<NT>(a, t0, ntok, dest_s);
}

template <int U, bool kMap, typename IdT, int kIds>
static void launch_fused_i(const PermuteArgs& a, const PermutePlan& p, size_t lds, hipStream_t stream) {
    if constexpr (U <= kPlainStoreMaxUnroll) {
        if (plain_row_stores(a)) {
            hipLaunchKernelGGL((permute_fused_kernel<kFusedThreads, U, false, kMap, IdT, kIds>),
                               dim3((unsigned)p.num_tiles), dim3(kFusedThreads), lds, stream, a, p.tokens_per_tile,
                               p.nbits);
            return;
        }
    }
    hipLaunchKernelGGL((permute_fused_kernel<kFusedThreads, U, true, kMap, IdT, kIds>), dim3((unsigned)p.num_tiles),
                       dim3(kFusedThreads), lds, stream, a, p.tokens_per_tile, p.nbits);
}

// Id batches per thread: the fewest of 1, 4, 16 or 32 that cover N * topk rows
// (decode N=1 permute 5.33 -> 4.70 us against always 32; Mixtral shape, 16
// batches, 18.97 -> 18.77 us).
template <int U, bool kMap, typename IdT>
static void launch_fused_v(const PermuteArgs& a, const PermutePlan& p, hipStream_t stream) {
    const size_t lds = fused_lds_bytes(a.num_buckets, p.tile_rows, map_entries(a));
    constexpr int kMaxIds = kFusedMaxRows / kFusedThreads;
    if (p.rows <= kFusedThreads) launch_fused_i<U, kMap, IdT, 1>(a, p, lds, stream);
    else if (p.rows <= 4 * kFusedThreads) launch_fused_i<U, kMap, IdT, 4>(a, p, lds, stream);
    else if (p.rows <= 16 * kFusedThreads) launch_fused_i<U, kMap, IdT, 16>(a, p, lds, stream);
    else launch_fused_i<U, kMap, IdT, kMaxIds>(a, p, lds, stream);
}

template <int U>
static void launch_fused_u(const PermuteArgs& a, const PermutePlan& p, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_fused_v<U, kMap, IdT>(a, p, stream);
    });
}

hipError_t launch_permute_fused(const PermuteArgs& a, const PermutePlan& p, int u, hipStream_t stream) {
#define MOE_FUSED(U) launch_fused_u<U>(a, p, stream)
    MOE_DISPATCH_U(u, MOE_FUSED)
#undef MOE_FUSED
    return hipGetLastError();
}

}  // namespace moe
