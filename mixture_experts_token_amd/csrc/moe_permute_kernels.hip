// moe_permute_kernels.hip -- gfx950 (CDNA4) kernels for MoE token permute / unpermute.
//
// What is computed: vLLM PR #14568, "permute/unpermute kernel for moe
// optimization", PR description (expand + order tokens per expert, then fold
// the expanded expert output back per token with topk_weight); buffer layout
// per the prhub summary of vLLM PR #43014, section "key code snippets"
// (MoEPermuteScratch).
//
// The path moves bytes and does no matrix arithmetic, so there is no MFMA
// here: the kernels are built around 64-lane wavefronts, LDS and 16-byte
// vector memory operations.
//
// Stable order without atomics deciding it: inside a wavefront, the lanes
// holding the same expert id are found with one ballot per id bit, and a
// row's rank among them is the count of such lanes below it (mbcnt).  Waves
// own contiguous row spans and keep per-expert running counts in LDS; a scan
// over waves, then over tiles, turns these into global positions.  Counts that
// only need a total (not an order) use LDS atomics, whose order cannot change
// an integer sum.  Every result is therefore deterministic.
//
// Row movement is token-major: each token row is read once and written to its
// topk destinations, so HBM reads equal the algorithmic N*H bytes.  A wave
// issues the loads of its first row chunk before the index work starts, and
// barriers inside the kernels order LDS only, so those loads stay in flight
// while the ranks are computed; the copy loop then double-buffers (loads of
// the next chunk are in flight while the current chunk is stored).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// Wavefront / workgroup helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Lanes of this wavefront whose `key` equals the calling lane's key, among
// the lanes with `live` set.  Meaningful only on live lanes.
__device__ __forceinline__ uint64_t lanes_with_same_key(int key, bool live, int nbits) {
    uint64_t m = __ballot(live);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = __ballot(live && bit);
        m &= bit ? ones : ~ones;
    }
    return m;
}

__device__ __forceinline__ int wave_index() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveSize));
}

// Workgroup barrier that orders LDS only.  Global loads issued before it stay
// in flight (no wait on the vector-memory counter); nothing in these kernels
// communicates through global memory inside one launch.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------------------------
// Sort keys.  Without a map a row's key is its expert id.  With a local-expert
// map (expert parallelism: the offsets cover this rank's experts only) the key
// is the expert's local id, and a row whose expert lives on another rank gets
// no key: it is not ranked, copied or counted, and its inverse index is -1.
// ----------------------------------------------------------------------------
constexpr int kRemoteKey = -1;  // expert on another rank
constexpr int kBadKey = -2;     // id outside [0, E), or a map entry outside [-1, B)

// kMap: the kernel was built for a map (map_s is its LDS copy); otherwise
// map_s is not read and the key is the expert id.
template <bool kMap>
__device__ __forceinline__ int bucket_of(int id, int E, const int* map_s, int B) {
    if ((unsigned)id >= (unsigned)E) return kBadKey;
    if constexpr (!kMap) {
        return id;
    } else {
        const int m = map_s[id];
        if (m == -1) return kRemoteKey;
        return (unsigned)m < (unsigned)B ? m : kBadKey;
    }
}

// Expert id of expanded row r.  int64 ids outside [0, 2^31) become -1, which
// every caller treats as out of range: a value is never truncated into range.
__device__ __forceinline__ int load_id(const int32_t* ids, int64_t r) { return ids[r]; }
__device__ __forceinline__ int load_id(const int64_t* ids, int64_t r) {
    const int64_t v = ids[r];
    return (v >= 0 && v <= INT32_MAX) ? (int)v : -1;
}

// The map, read into registers with the other early index loads (before any
// row prefetch: the vector-memory counter retires in issue order) and written
// to LDS before the first barrier.  Empty without a map.
template <int NT, bool kMap>
struct MapStage {
    static constexpr int kPer = kMap ? (kMaxExperts + NT - 1) / NT : 0;
    int v[kPer > 0 ? kPer : 1];

    __device__ __forceinline__ void load(const PermuteArgs& a) {
        const int E = a.num_experts;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = (int)threadIdx.x + j * NT;
            v[j] = a.expert_map[i < E ? i : E - 1];
        }
    }

    // Returns the LDS copy (null without a map).
    __device__ __forceinline__ const int* store(const PermuteArgs& a, int* map_s) const {
        if constexpr (!kMap) return nullptr;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = (int)threadIdx.x + j * NT;
            if (i < a.num_experts) map_s[i] = v[j];
        }
        return map_s;
    }
};

// Exclusive prefix sum of data[0..n) in LDS, in place; returns the total.
// Every thread of the workgroup must call it.  tmp: NT/64 ints of LDS.
template <int NT>
__device__ int block_exclusive_scan(int* data, int n, int* tmp) {
    constexpr int W = NT / kWaveSize;
    const int tid = threadIdx.x, lane = tid % kWaveSize, w = tid / kWaveSize;
    const int per = (n + NT - 1) / NT;
    const int beg = min(tid * per, n), end = min(beg + per, n);
    int s = 0;
    for (int i = beg; i < end; ++i) s += data[i];
    int x = s;
#pragma unroll
    for (int d = 1; d < kWaveSize; d <<= 1) {
        const int y = __shfl_up(x, d, kWaveSize);
        if (lane >= d) x += y;
    }
    if (lane == kWaveSize - 1) tmp[w] = x;
    lds_barrier();
    int before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) {
        const int c = tmp[v];
        before += v < w ? c : 0;
        total += c;
    }
    int run = before + x - s;
    for (int i = beg; i < end; ++i) {
        const int c = data[i];
        data[i] = run;
        run += c;
    }
    lds_barrier();
    return total;
}

// ----------------------------------------------------------------------------
// Stable ranks within one tile of expanded rows, keys already in LDS.
//
// key_s[i] is the bucket of tile row i, or -1 for a row without one (an
// out-of-range id or a remote expert; such rows get no rank).  Wave w owns rows [w*span, (w+1)*span) and
// walks them 64 at a time, so a row's rank is (rows of its expert in earlier
// waves) + (rows of its expert earlier in its own wave).  On return, after a
// barrier:
//   rank_s[i] rank of row i among the tile's rows with the same key
//   cnt_s[e]  rows of the tile with key e (B keys)
// wave_s (NT/64 * B ints) must be zero on entry; it is clobbered.
// ----------------------------------------------------------------------------
template <int NT>
__device__ void rank_tile(const int* key_s, int tile_rows, int B, int nbits, int* rank_s, int* wave_s, int* cnt_s) {
    constexpr int W = NT / kWaveSize;
    const int w = wave_index();
    const int lane = threadIdx.x % kWaveSize;
    const int span = (tile_rows + NT - 1) / NT * kWaveSize;
    const int beg = w * span;
    const int end = min(beg + span, tile_rows);
    int* run = wave_s + w * B;
    for (int base = beg; base < end; base += kWaveSize) {
        const int i = base + lane;
        const int key = i < end ? key_s[i] : -1;
        const bool ok = key >= 0;
        const uint64_t same = lanes_with_same_key(key, ok, nbits);
        const int below = lanes_below(same);
        if (ok) {
            const int r = run[key];
            rank_s[i] = r + below;
            if (below == 0) run[key] = r + (int)__popcll(same);
        } else if (i < end) {
            rank_s[i] = 0;
        }
    }
    lds_barrier();
    for (int e = threadIdx.x; e < B; e += NT) {
        int s = 0;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            const int c = wave_s[v * B + e];
            wave_s[v * B + e] = s;
            s += c;
        }
        cnt_s[e] = s;
    }
    lds_barrier();
    for (int i = threadIdx.x; i < tile_rows; i += NT) {
        const int key = key_s[i];
        if (key >= 0) rank_s[i] += wave_s[(i / span) * B + key];
    }
    lds_barrier();
}

// ----------------------------------------------------------------------------
// Token-major row copy of one tile.  Work items are (token of the tile, chunk
// of U*64 16-byte vectors); wave w takes items w, w+W, ...  dest_s[tl*topk+k]
// is the permuted row of the tile's token tl, slot k.
// ----------------------------------------------------------------------------
template <int U, bool kNTStore, bool kSparse, typename IdT>
struct TileCopy {
    const u32x4* __restrict__ src;  // first row of the tile
    u32x4* __restrict__ dst;        // permuted_hidden_states
    const IdT* ids;                 // topk_ids of the tile's first token
    const int32_t* emap;            // expert map (kSparse)
    int64_t rv;                     // row length in vectors
    int64_t rows_total;             // N * topk
    int nchunks;
    int items;
    int K;
    int E;
    int lane;

    __device__ TileCopy(const PermuteArgs& a, int64_t t0, int ntok)
        : src(reinterpret_cast<const u32x4*>(a.hidden_states) + t0 * a.row_vecs),
          dst(reinterpret_cast<u32x4*>(a.permuted_hidden_states)),
          ids(static_cast<const IdT*>(a.topk_ids) + t0 * a.topk),
          emap(a.expert_map),
          rv(a.row_vecs),
          rows_total(a.num_tokens * a.topk),
          nchunks((int)((a.row_vecs + U * kWaveSize - 1) / (U * kWaveSize))),
          items(ntok * (int)((a.row_vecs + U * kWaveSize - 1) / (U * kWaveSize))),
          K(a.topk),
          E(a.num_experts),
          lane((int)(threadIdx.x % kWaveSize)) {}

    __device__ __forceinline__ void load_rows(int it, u32x4 (&v)[U], bool live) const {
        const int tl = it / nchunks;
        const int64_t base = (int64_t)(it - tl * nchunks) * (U * kWaveSize) + lane;
        const u32x4* s = src + tl * rv;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWaveSize;
            v[u] = (live && idx < rv) ? __builtin_nontemporal_load(s + idx) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Loads item it's chunk.  kSparse (a local-expert map: some rows have no
    // destination): a token with no destination is not read at all.
    __device__ __forceinline__ void load(int it, u32x4 (&v)[U], const int* dest_s) const {
        bool live = true;
        if constexpr (kSparse) {
            const int tl = it / nchunks;
            live = false;
            for (int k = 0; k < K; ++k) live |= (uint32_t)dest_s[tl * K + k] < (uint64_t)rows_total;
        }
        load_rows(it, v, live);
    }

    // Early load of wave w's first item, before the destinations exist.  With
    // kSparse the token is read only if one of its experts is local; its ids
    // and their map entries sit at wave-uniform addresses, so those reads go
    // through the scalar path and leave the vector-memory counter to the row
    // loads.  A token with nothing local is not read (none of its chunks is
    // stored).
    __device__ __forceinline__ void prefetch(int w, u32x4 (&v)[U]) const {
        if (rv == 0 || w >= items) return;
        bool live = true;
        if constexpr (kSparse) {
            // Eight ids, then their eight map entries, per round trip (clamped
            // addresses, so every read is in bounds and none waits on a branch).
            const int tl = __builtin_amdgcn_readfirstlane(w / nchunks);
            const IdT* tid = ids + tl * K;
            live = false;
            int any = 0;
            for (int k0 = 0; k0 < K; k0 += 8) {
                int id[8], m[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) id[q] = load_id(tid, min(k0 + q, K - 1));
#pragma unroll
                for (int q = 0; q < 8; ++q) m[q] = emap[min((unsigned)id[q], (unsigned)(E - 1))];
#pragma unroll
                for (int q = 0; q < 8; ++q) any |= (int)((unsigned)id[q] < (unsigned)E) & (int)(m[q] >= 0);
            }
            live = any != 0;
        }
        load_rows(w, v, live);
    }

    __device__ __forceinline__ void store(int it, const u32x4 (&v)[U], const int* dest_s) const {
        const int tl = it / nchunks;
        const int64_t base = (int64_t)(it - tl * nchunks) * (U * kWaveSize) + lane;
        for (int k = 0; k < K; ++k) {
            const int d = dest_s[tl * K + k];
            if ((uint32_t)d >= (uint64_t)rows_total) continue;  // never taken when the ranks are right
            u32x4* o = dst + (int64_t)d * rv;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = base + u * kWaveSize;
                if (idx < rv) {
                    if constexpr (kNTStore)
                        __builtin_nontemporal_store(v[u], o + idx);
                    else
                        o[idx] = v[u];
                }
            }
        }
    }
};

// Store every item of wave w, starting from `cur` (already loaded for item w),
// loading item it+W while item it is stored.
// cur already holds the wave's first item (TileCopy::prefetch).
template <int U, int NT, bool kNTStore, bool kSparse, typename IdT>
__device__ __forceinline__ void copy_items_pipelined(const TileCopy<U, kNTStore, kSparse, IdT>& tc, u32x4 (&cur)[U],
                                                     const int* dest_s) {
    constexpr int W = NT / kWaveSize;
    for (int it = wave_index(); it < tc.items; it += W) {
        u32x4 nxt[U];
        const bool more = it + W < tc.items;
        if (more) tc.load(it + W, nxt, dest_s);
        tc.store(it, cur, dest_s);
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
    }
}

template <int NT>
__device__ __forceinline__ void copy_tile_scales(const PermuteArgs& a, int64_t t0, int ntok, const int* dest_s) {
    if (a.token_scale == nullptr) return;
    const int K = a.topk;
    const int64_t rows_total = a.num_tokens * K;
    for (int i = threadIdx.x; i < ntok * K; i += NT) {
        const int d = dest_s[i];
        if ((uint32_t)d < (uint64_t)rows_total) a.permuted_scale[d] = a.token_scale[t0 + i / K];
    }
}

// ----------------------------------------------------------------------------
// Tile phases shared by the fused and coarse schedules.  A tile is a run of
// whole tokens (T expanded rows from row0); wave w ranks tile rows
// [w*span, w*span + span), span = ceil(T / NT) * 64, at most kB batches of 64.
// ----------------------------------------------------------------------------

// Expert ids of this wave's tile rows (issued early, independent loads);
// tile_keys_to_buckets turns them into sort keys once the map is in LDS.
template <int kB, typename IdT>
__device__ __forceinline__ void load_tile_keys(const IdT* __restrict__ ids, int row0, int T, int span, int w,
                                               int lane, int (&tkey)[kB]) {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
        const int i = w * span + b * kWaveSize + lane;
        tkey[b] = load_id(ids, row0 + (i < T ? i : T - 1));
    }
}

template <bool kMap, int kB>
__device__ __forceinline__ void tile_keys_to_buckets(int (&tkey)[kB], int E, const int* map_s, int B) {
#pragma unroll
    for (int b = 0; b < kB; ++b) tkey[b] = bucket_of<kMap>(tkey[b], E, map_s, B);
}

__device__ __forceinline__ bool own_row(int b, int i, int T, int span, int w) {
    return b * kWaveSize < span && i < T && i < w * span + span;
}

// Stable ranks of this wave's tile rows among the wave's rows with the same
// key (ballot match + mbcnt); the lowest lane of each equal-key group adds
// the group size to the wave's running count run[key].  Rows without a key
// are not ranked.  Returns the number of bad ids or map entries among the
// wave's rows (this lane's share).  Without a map tkey holds the raw expert
// ids (valid in [0, E)); with one, the keys from tile_keys_to_buckets.
template <bool kMap, int kB>
__device__ __forceinline__ int rank_own_rows(const int (&tkey)[kB], int T, int span, int E, int nbits, int w,
                                             int lane, int* run, int (&trank)[kB]) {
    int nbad = 0;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
        const int base = w * span + b * kWaveSize;
        trank[b] = 0;
        if (b * kWaveSize < span && base < T) {  // wave-uniform
            const int i = base + lane;
            const bool in_tile = own_row(b, i, T, span, w);
            bool ok;
            if constexpr (kMap) {
                ok = in_tile && tkey[b] >= 0;
                nbad += (in_tile && tkey[b] == kBadKey) ? 1 : 0;
            } else {
                ok = in_tile && (unsigned)tkey[b] < (unsigned)E;
                nbad += (in_tile && !ok) ? 1 : 0;
            }
            const uint64_t same = lanes_with_same_key(tkey[b], ok, nbits);
            const int below = lanes_below(same);
            if (ok) {
                const int c = run[tkey[b]];
                trank[b] = c + below;
                if (below == 0) run[tkey[b]] = c + (int)__popcll(same);
            }
        }
    }
    return nbad;
}

// Per bucket e of B (kPer consecutive buckets per thread): turn the per-wave
// counts wave_s[v*B + e] into prefixes over waves, take the bucket's total
// rows total_of(e, rows_in_tile), scan the totals over buckets (one barrier)
// into expert_first_token_offset[0..B] (written when write_off), and store the
// tile's base in each bucket, offset + before_of(e), into base_s[e].  Each
// bucket is read and written by one thread only, so base_s may alias
// before_of's data.
template <int NT, int kPer, class TotalFn, class BeforeFn>
__device__ __forceinline__ void expert_bases(int B, int* wave_s, int* base_s, int* scan_tmp, int64_t* off_out,
                                             bool write_off, TotalFn total_of, BeforeFn before_of) {
    constexpr int W = NT / kWaveSize;
    const int w = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;
    int tot[kPer];
    int s = 0;
    const int e0 = (int)threadIdx.x * kPer;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = e0 + q;
        tot[q] = 0;
        if (e < B) {
            int c = 0;
#pragma unroll
            for (int v = 0; v < W; ++v) {
                const int x = wave_s[v * B + e];
                wave_s[v * B + e] = c;
                c += x;
            }
            tot[q] = total_of(e, c);
        }
        s += tot[q];
    }
    int x = s;
#pragma unroll
    for (int d = 1; d < kWaveSize; d <<= 1) {
        const int y = __shfl_up(x, d, kWaveSize);
        if (lane >= d) x += y;
    }
    if (lane == kWaveSize - 1) scan_tmp[w] = x;
    lds_barrier();
    int excl = x - s, total = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) {
        const int c = scan_tmp[v];
        excl += v < w ? c : 0;
        total += c;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = e0 + q;
        if (e < B) {
            if (write_off) off_out[e] = excl;
            base_s[e] = excl + before_of(e);
            excl += tot[q];
        }
    }
    if (write_off && threadIdx.x == 0) off_out[B] = total;
}

// Destinations of this wave's tile rows: tile base + rows of the same key in
// earlier waves + rank within the wave; -1 for a row of a remote expert.
template <bool kMap, int kB>
__device__ __forceinline__ void write_dests(const PermuteArgs& a, const int (&tkey)[kB], const int (&trank)[kB],
                                            int row0, int T, int span, int B, int w, int lane, const int* base_s,
                                            const int* wave_s, int* dest_s) {
    const int64_t R = a.num_tokens * a.topk;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
        const int i = w * span + b * kWaveSize + lane;
        if (own_row(b, i, T, span, w)) {
            const int key = tkey[b];
            if constexpr (kMap) {
                if (key < 0) {  // remote expert (bad keys never get here)
                    dest_s[i] = -1;
                    a.inv_permuted_idx[row0 + i] = -1;
                    continue;
                }
            }
            const int dest = base_s[key] + wave_s[w * B + key] + trank[b];
            dest_s[i] = dest;
            a.inv_permuted_idx[row0 + i] = dest;
            if ((uint32_t)dest < (uint64_t)R) a.permuted_idx[dest] = row0 + i;
        }
    }
}

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
    const int64_t tile = blockIdx.x;
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
        int x = s;
#pragma unroll
        for (int d = 1; d < kWaveSize; d <<= 1) {
            const int y = __shfl_up(x, d, kWaveSize);
            if (lane >= d) x += y;
        }
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
    const int64_t tile = blockIdx.x;
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

__global__ void fill_offsets_kernel(int64_t* off, int n, int64_t value) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) off[i] = value;
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
// Launchers
// ----------------------------------------------------------------------------
// Vectors per lane in the permute row copy: up to 8 while a row has few
// copies (2-way fan-out measured best with full-row chunks), up to 4 for
// 4-way and wider fan-out (measured slightly faster: more waves in flight).
static constexpr int kCopyUnrolls[] = {8, 7, 6, 5, 4, 3, 2, 1};
static constexpr int kCopyUnrollsWideFanout[] = {4, 3, 2, 1};

hipError_t launch_fill_offsets(int64_t* off, int num_experts, int64_t value, hipStream_t stream) {
    hipLaunchKernelGGL(fill_offsets_kernel, dim3(1), dim3(256), 0, stream, off, num_experts + 1, value);
    return hipGetLastError();
}

// Row stores: plain stores when each row fans out to many destinations and
// the permuted output is large (measured faster for 8-way fan-out at 256 MiB
// and above); non-temporal otherwise (faster for 2-way fan-out and for small
// outputs).  Measured with buffer rotation well beyond the last-level cache.
static constexpr int kPlainStoreMinTopk = 4;
static constexpr int64_t kPlainStoreMinBytes = int64_t(32) << 20;

static bool plain_row_stores(const PermuteArgs& a) {
    return a.topk >= kPlainStoreMinTopk && a.num_tokens * a.topk * a.row_vecs * 16 >= kPlainStoreMinBytes;
}

// Plain stores come with topk >= 4, whose row chunks are at most 4 vectors
// per lane (kCopyUnrollsWideFanout), so wider chunks are built for
// non-temporal stores only.
static constexpr int kPlainStoreMaxUnroll = kCopyUnrollsWideFanout[0];
static_assert(kPlainStoreMinTopk >= 4, "plain row stores only where the wide-fan-out chunk widths apply");

static int map_entries(const PermuteArgs& a) { return a.expert_map != nullptr ? a.num_experts : 0; }

// The map and the id type are compile-time parameters of every permute
// kernel, so the plain int32 permute carries none of their code.  f receives
// std::integral_constant<bool, map> and a null `const IdT*` naming the id type.
template <class F>
static void with_variant(const PermuteArgs& a, F&& f) {
    if (a.expert_map != nullptr) {
        if (a.ids64) f(std::true_type{}, static_cast<const int64_t*>(nullptr));
        else f(std::true_type{}, static_cast<const int32_t*>(nullptr));
    } else {
        if (a.ids64) f(std::false_type{}, static_cast<const int64_t*>(nullptr));
        else f(std::false_type{}, static_cast<const int32_t*>(nullptr));
    }
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

template <int U, bool kMap, typename IdT>
static void launch_scatter_v(const PermuteArgs& a, const PermutePlan& p, const int32_t* rank_ws,
                             const int32_t* tile_base, const int32_t* total, hipStream_t stream) {
    const size_t lds = scatter_lds_bytes(a.num_buckets, p.tile_rows, map_entries(a));
    if constexpr (U <= kPlainStoreMaxUnroll) {
        if (plain_row_stores(a)) {
            hipLaunchKernelGGL((permute_scatter_kernel<kScatterThreads, U, false, kMap, IdT>),
                               dim3((unsigned)p.num_tiles), dim3(kScatterThreads), lds, stream, a, p.tokens_per_tile,
                               p.num_tiles, rank_ws, tile_base, total);
            return;
        }
    }
    hipLaunchKernelGGL((permute_scatter_kernel<kScatterThreads, U, true, kMap, IdT>), dim3((unsigned)p.num_tiles),
                       dim3(kScatterThreads), lds, stream, a, p.tokens_per_tile, p.num_tiles, rank_ws, tile_base,
                       total);
}

#define MOE_VARIANT_TYPES                                 \
    constexpr bool kMap = decltype(map_tag)::value;       \
    using IdT = std::remove_const_t<std::remove_pointer_t<decltype(id_tag)>>

template <int U>
static void launch_fused_u(const PermuteArgs& a, const PermutePlan& p, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_fused_v<U, kMap, IdT>(a, p, stream);
    });
}

template <int U>
static void launch_coarse_u(const PermuteArgs& a, const PermutePlan& p, const int32_t* hist, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_coarse_v<U, kMap, IdT>(a, p, hist, stream);
    });
}

template <int U>
static void launch_scatter_u(const PermuteArgs& a, const PermutePlan& p, const int32_t* rank_ws,
                             const int32_t* tile_base, const int32_t* total, hipStream_t stream) {
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        launch_scatter_v<U, kMap, IdT>(a, p, rank_ws, tile_base, total, stream);
    });
}

#define MOE_DISPATCH_U(u, CALL) \
    switch (u) {                \
        case 8: CALL(8); break; \
        case 7: CALL(7); break; \
        case 6: CALL(6); break; \
        case 5: CALL(5); break; \
        case 4: CALL(4); break; \
        case 3: CALL(3); break; \
        case 2: CALL(2); break; \
        default: CALL(1); break; \
    }

hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t stream) {
    const int B = a.num_buckets;
    const int M = map_entries(a);
    const int u = a.topk >= 4 ? choose_unroll(a.row_vecs, kCopyUnrollsWideFanout, 4)
                              : choose_unroll(a.row_vecs, kCopyUnrolls, 8);
    if (p.fused) {
#define MOE_FUSED(U) launch_fused_u<U>(a, p, stream)
        MOE_DISPATCH_U(u, MOE_FUSED)
#undef MOE_FUSED
        return hipGetLastError();
    }
    char* ws = static_cast<char*>(workspace);
    if (p.coarse) {
        int32_t* hist = reinterpret_cast<int32_t*>(ws);
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
    int32_t* rank_ws = reinterpret_cast<int32_t*>(ws + p.ws_rank);
    int32_t* tile_hist = reinterpret_cast<int32_t*>(ws + p.ws_tile_hist);
    int32_t* total = reinterpret_cast<int32_t*>(ws + p.ws_total);
    with_variant(a, [&](auto map_tag, auto id_tag) {
        MOE_VARIANT_TYPES;
        hipLaunchKernelGGL((permute_rank_tiles_kernel<kRankThreads, kMap, IdT>), dim3((unsigned)p.num_tiles),
                           dim3(kRankThreads), rank_lds_bytes(B, p.tile_rows, M), stream, a, p.tokens_per_tile,
                           p.nbits, p.num_tiles, rank_ws, tile_hist);
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

template <bool kBF16, int KC, int U, int G>
static hipError_t launch_unpermute_t(const UnpermuteArgs& a, hipStream_t stream) {
    const int64_t nchunks = (a.row_vecs + U * kWaveSize - 1) / (U * kWaveSize);
    const int64_t items = a.num_tokens * nchunks;
    const int64_t blocks_needed = (items + 3) / 4;
    const int64_t blocks = blocks_needed < kMaxGridBlocks ? blocks_needed : kMaxGridBlocks;
    hipLaunchKernelGGL((unpermute_kernel<kBF16, KC, U, G>), dim3((unsigned)blocks), dim3(256), 0, stream,
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
