// moe_permute_staged.hip -- staged permute schedule (three kernels: rank tiles, scan, scatter).
// What is computed and how ranks stay stable: see moe_permute_device.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

// ----------------------------------------------------------------------------
// Staged permute, kernel 1: per tile, stable ranks and the bucket histogram.
// rank_ws[r] = rank of row r within its tile; tile_hist[b][tile] = count,
// tile_hist[B][tile] = rows with a bad id or map entry.
// ----------------------------------------------------------------------------
template <int NT, bool kMap, typename IdT>
__global__ __launch_bounds__(NT) void permute_rank_tiles_kernel(PermuteArgs a, int tokens_per_tile, int nbits,
                                                                int64_t num_tiles, int32_t* rank_ws,
                                                                int32_t* tile_hist) {
    constexpr int W = NT / kWaveSize;
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int B = a.num_buckets;
    const int K = a.topk;
    const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;  // 2-D grid (staged_grid)
    if (tile >= num_tiles) return;
    const int64_t t0 = tile * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int64_t row0 = t0 * K;
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;

    int* cnt_s = smem;                    // [B]
    int* wave_s = cnt_s + B;              // [W * B]
    int* key_s = wave_s + W * B;          // [tile_cap]
    int* rank_s = key_s + tile_cap;       // [tile_cap]
    int* misc_s = rank_s + tile_cap;      // [16]
    int* map_w = misc_s + 16;             // [E] with a map

    for (int i = threadIdx.x; i < (1 + W) * B; i += NT) smem[i] = 0;
    if (threadIdx.x < 16) misc_s[threadIdx.x] = 0;
    if constexpr (kMap)
        for (int e = threadIdx.x; e < E; e += NT) map_w[e] = a.expert_map[e];
    lds_barrier();
    const int* map_s = map_w;
    int nbad = 0;
    for (int i = threadIdx.x; i < T; i += NT) {
        const int key = bucket_of<kMap>(load_id(static_cast<const IdT*>(a.topk_ids), row0 + i), E, map_s, B);
        nbad += key == kBadKey ? 1 : 0;
        key_s[i] = key >= 0 ? key : -1;
    }
    if (nbad) atomicAdd(&misc_s[0], nbad);
    lds_barrier();
    rank_tile<NT>(key_s, T, B, nbits, rank_s, wave_s, cnt_s);
    for (int i = threadIdx.x; i < T; i += NT) rank_ws[row0 + i] = rank_s[i];
    for (int e = threadIdx.x; e < B; e += NT) tile_hist[(int64_t)e * num_tiles + tile] = cnt_s[e];
    if (threadIdx.x == 0) tile_hist[(int64_t)B * num_tiles + tile] = misc_s[0];
}

// ----------------------------------------------------------------------------
// Staged permute, kernel 2: one workgroup per histogram row (an expert, or the
// bad-id row E).  The row's tile counts are loaded at once (P per thread,
// thread-contiguous), scanned in registers, then across the workgroup; the
// exclusive prefix goes back in place and the row total to total[e].
// ----------------------------------------------------------------------------
template <int NT, int P>
__global__ __launch_bounds__(NT) void permute_scan_tiles_kernel(int32_t* tile_hist, int64_t num_tiles,
                                                                int32_t* total) {
    __shared__ int tmp[NT / kWaveSize];
    const int tid = threadIdx.x;
    const int lane = tid % kWaveSize, w = tid / kWaveSize;
    int32_t* row = tile_hist + (int64_t)blockIdx.x * num_tiles;
    int carry = 0;
    for (int64_t base = 0; base < num_tiles; base += (int64_t)NT * P) {
        const int64_t first = base + (int64_t)tid * P;
        int v[P];
#pragma unroll
        for (int p = 0; p < P; ++p) v[p] = first + p < num_tiles ? row[first + p] : 0;
        int s = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = v[p];
            v[p] = s;  // exclusive within the thread
            s += c;
        }
        const int x = wave_inclusive_scan(s);
        if (lane == kWaveSize - 1) tmp[w] = x;
        lds_barrier();
        int before = carry, pass_total = 0;
#pragma unroll
        for (int q = 0; q < NT / kWaveSize; ++q) {
            const int c = tmp[q];
            before += q < w ? c : 0;
            pass_total += c;
        }
        before += x - s;
#pragma unroll
        for (int p = 0; p < P; ++p)
            if (first + p < num_tiles) row[first + p] = before + v[p];
        carry += pass_total;
        lds_barrier();  // tmp is reused by the next pass
    }
    if (tid == 0) total[blockIdx.x] = carry;
}

// ----------------------------------------------------------------------------
// Staged permute, kernel 3: offsets from the per-bucket totals, destinations
// from offset + tile base + rank, index scatter, and the row copy.
// ----------------------------------------------------------------------------
template <int NT, int U, bool kNTStore, bool kMap, typename IdT>
__global__ __launch_bounds__(NT) void permute_scatter_kernel(PermuteArgs a, int tokens_per_tile, int64_t num_tiles,
                                                             const int32_t* rank_ws, const int32_t* tile_base,
                                                             const int32_t* total) {
    constexpr int kE = (kMaxExperts + 1 + NT - 1) / NT;  // per-bucket values held per thread
    constexpr int kT = (kMaxTileRows + NT - 1) / NT;     // tile rows held per thread
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int B = a.num_buckets;
    const int K = a.topk;
    const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;  // 2-D grid (staged_grid)
    if (tile >= num_tiles) return;
    const int64_t t0 = tile * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int64_t row0 = t0 * K;
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;
    const int64_t R = a.num_tokens * K;

    // Independent index loads first, then the first row chunk of this wave
    // (the vector-memory counter retires in issue order).
    int tot[kE], tb[kE], key[kT], rk[kT];
#pragma unroll
    for (int j = 0; j < kE; ++j) {
        const int e = (int)threadIdx.x + j * NT;
        tot[j] = total[e <= B ? e : B];
        tb[j] = tile_base[(int64_t)(e < B ? e : B - 1) * num_tiles + tile];
    }
#pragma unroll
    for (int j = 0; j < kT; ++j) {
        const int i = (int)threadIdx.x + j * NT;
        const int64_t r = row0 + (i < T ? i : T - 1);
        key[j] = load_id(static_cast<const IdT*>(a.topk_ids), r);
        rk[j] = rank_ws[r];
    }
    MapStage<NT, kMap> ms;
    ms.load(a);
    const TileCopy<U, kNTStore, kMap, IdT> tc(a, t0, ntok);
    u32x4 cur[U];
    tc.prefetch(wave_index(), cur);

    int* off_s = smem;                // [B + 1] totals, then offsets
    int* base_s = off_s + (B + 1);    // [B]     this tile's base within each bucket
    int* dest_s = base_s + B;         // [tile_cap]
    int* misc_s = dest_s + tile_cap;  // [16]
    const int* map_s = ms.store(a, misc_s + 16);  // [E] with a map

#pragma unroll
    for (int j = 0; j < kE; ++j) {
        const int e = (int)threadIdx.x + j * NT;
        if (e <= B) off_s[e] = tot[j];
        if (e < B) base_s[e] = tb[j];
    }
    lds_barrier();
    if (off_s[B] != 0) {  // a bad id or map entry: report through the offsets, write nothing else
        if (tile == 0)
            for (int e = threadIdx.x; e <= B; e += NT) a.expert_first_token_offset[e] = -1;
        return;
    }
    const int rows_total = block_exclusive_scan<NT>(off_s, B, misc_s);
    if (tile == 0) {
        for (int e = threadIdx.x; e < B; e += NT) a.expert_first_token_offset[e] = off_s[e];
        if (threadIdx.x == 0) a.expert_first_token_offset[B] = rows_total;
    }
#pragma unroll
    for (int j = 0; j < kT; ++j) {
        const int i = (int)threadIdx.x + j * NT;
        if (i >= T) continue;
        int e;
        if constexpr (kMap) {
            e = bucket_of<true>(key[j], E, map_s, B);  // never bad here (no bad-id count)
            if (e < 0) {  // remote expert
                dest_s[i] = -1;
                a.inv_permuted_idx[row0 + i] = -1;
                continue;
            }
        } else {
            e = min(max(key[j], 0), E - 1);  // all ids are in range here (no bad-id count)
        }
        const int dest = off_s[e] + base_s[e] + rk[j];
        dest_s[i] = dest;
        a.inv_permuted_idx[row0 + i] = dest;
        if ((uint32_t)dest < (uint64_t)R) a.permuted_idx[dest] = (int32_t)(row0 + i);
    }
    lds_barrier();
    if (a.row_vecs > 0) copy_items_pipelined<U, NT, kNTStore, kMap, IdT>(tc, cur, dest_s);
    copy_tile_scales<NT>(a, t0, ntok, dest_s);
}

template <int U, bool kMap, typename IdT>
static void launch_scatter_v(const PermuteArgs& a, const PermutePlan& p, const int32_t* rank_ws,
                             const int32_t* tile_base, const int32_t* total, hipStream_t stream) {
    const size_t lds = scatter_lds_bytes(a.num_buckets, p.tile_rows, map_entries(a));
    unsigned gx, gy;
    staged_grid(p.num_tiles, gx, gy);
    if constexpr (U <= kPlainStoreMaxUnroll) {
        if (plain_row_stores(a)) {
            hipLaunchKernelGGL((permute_scatter_kernel<kScatterThreads, U, false, kMap, IdT>), dim3(gx, gy),
                               dim3(kScatterThreads), lds, stream, a, p.tokens_per_tile, p.num_tiles, rank_ws,
                               tile_base, total);
            return;
        }
    }
    hipLaunchKernelGGL((permute_scatter_kernel<kScatterThreads, U, true, kMap, IdT>), dim3(gx, gy),
                       dim3(kScatterThreads), lds, stream, a, p.tokens_per_tile, p.num_tiles, rank_ws, tile_base,
                       total);
}

template <int U>
static void launch_scatter_u(const PermuteArgs& a, const PermutePlan& p, const int32_t* rank_ws,
                             const int32_t* tile_base, const int32_t* total, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_scatter_v<U, kMap, IdT>(a, p, rank_ws, tile_base, total, stream);
    });
}

hipError_t launch_permute_staged(const PermuteArgs& a, const PermutePlan& p, void* workspace, int u,
                                 hipStream_t stream) {
    const int B = a.num_buckets;
    const int M = map_entries(a);
    char* ws = static_cast<char*>(workspace);
    int32_t* rank_ws = reinterpret_cast<int32_t*>(ws + p.ws_rank);
    int32_t* tile_hist = reinterpret_cast<int32_t*>(ws + p.ws_tile_hist);
    int32_t* total = reinterpret_cast<int32_t*>(ws + p.ws_total);
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        unsigned gx, gy;
        staged_grid(p.num_tiles, gx, gy);
        hipLaunchKernelGGL((permute_rank_tiles_kernel<kRankThreads, kMap, IdT>), dim3(gx, gy), dim3(kRankThreads),
                           rank_lds_bytes(B, p.tile_rows, M), stream, a, p.tokens_per_tile, p.nbits, p.num_tiles,
                           rank_ws, tile_hist);
    });
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((permute_scan_tiles_kernel<kScanThreads, kScanPerThread>), dim3((unsigned)(B + 1)),
                       dim3(kScanThreads), 0, stream, tile_hist, p.num_tiles, total);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
#define MOE_SCATTER(U) launch_scatter_u<U>(a, p, rank_ws, tile_hist, total, stream)
    MOE_DISPATCH_U(u, MOE_SCATTER)
#undef MOE_SCATTER
    return hipGetLastError();
}

}  // namespace moe
