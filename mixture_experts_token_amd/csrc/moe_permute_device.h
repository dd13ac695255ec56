// moe_permute_device.h -- device helpers shared by the gfx950 (CDNA4) permute kernels.
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
#pragma once

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

// Inclusive prefix sum over the 64 lanes of a wave (every lane active), by
// DPP moves: shifts by 1, 2, 4 and 8 lanes within each 16-lane row, then lane
// 15 of rows 0 and 2 added into rows 1 and 3, and lane 31 into rows 2 and 3.
// Lanes whose source lies outside the row (or whose row the mask leaves out)
// add 0.  Six dependent VALU steps; the same sum through lane shuffles took six
// LDS-crossbar round trips.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
    return x;
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
// Wave schedule index pass (decode sizes, no expert map): one wave holds all R
// <= 64 * kPer expert ids of the call (id[j] is row j * 64 + lane; rows past R
// hold any valid load and are ignored) and computes the whole index itself:
//   * stable ranks: rows walked in batches of 64 in ascending order; inside a
//     batch the lanes with the same expert are found with one ballot per id
//     bit and a row's rank is the count of such lanes below it (mbcnt) plus
//     the rows of its expert in earlier batches (a running count in LDS,
//     advanced by the lowest lane of each equal-key group);
//   * the running counts end as the rows per expert; their exclusive scan
//     (DPP lane moves) gives the offsets, and destination = offset + rank.
// run: LDS [E]; dest_s: LDS [R], filled with each row's destination.  When
// `writer`, the offsets, permuted_idx, inv_permuted_idx (and, with kScale,
// the per-token scales sc moved to their rows) are written.  Returns false
// when an id is outside [0, E): the writer has then set every offset to -1
// and nothing else is written.  The same answer in every wave, since every
// wave sees every id.
// ----------------------------------------------------------------------------
// Orders the LDS accesses of this wave (the compiler must not move them across
// it; the hardware completes one wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local"); }

template <int kPer, bool kScale>
__device__ __forceinline__ bool wave_index_pass(int E, int R, int nbits, const int (&id)[kPer],
                                                const float (&sc)[kPer], int* run, int* dest_s, bool writer,
                                                int64_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                int32_t* __restrict__ inv, float* __restrict__ pscale) {
    const int lane = (int)(threadIdx.x % kWaveSize);
    for (int e = lane; e < E; e += kWaveSize) run[e] = 0;
    wave_lds_fence();

    // Stable ranks, batch by batch; run[e] ends as the rows of expert e.
    int rank[kPer];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        rank[j] = 0;
        if (j * kWaveSize < R) {  // wave-uniform
            const int r = j * kWaveSize + lane;
            const bool live = r < R;
            const bool ok = live && (unsigned)id[j] < (unsigned)E;
            bad |= live && !ok;
            const uint64_t same = lanes_with_same_key(id[j], ok, nbits);
            const int below = lanes_below(same);
            if (ok) {
                const int c = run[id[j]];
                rank[j] = c + below;
                if (below == 0) run[id[j]] = c + (int)__popcll(same);
            }
            wave_lds_fence();
        }
    }
    if (__ballot(bad) != 0) {
        if (writer)
            for (int e = lane; e <= E; e += kWaveSize) offsets[e] = -1;
        return false;
    }

    // Exclusive scan of the counts in place: lane l owns experts [l*per, l*per + per).
    const int per = (E + kWaveSize - 1) / kWaveSize;
    const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
    int s = 0;
    for (int e = e0; e < e1; ++e) s += run[e];
    const int x = wave_inclusive_scan(s);
    int acc = x - s;
    for (int e = e0; e < e1; ++e) {
        const int c = run[e];
        run[e] = acc;
        if (writer) offsets[e] = acc;
        acc += c;
    }
    if (writer && lane == 0) offsets[E] = R;
    wave_lds_fence();

#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int r = j * kWaveSize + lane;
        if (r < R) {
            const int d = run[id[j]] + rank[j];
            dest_s[r] = d;
            if (writer) {
                inv[r] = d;
                perm[d] = r;
                if constexpr (kScale) pscale[d] = sc[j];
            }
        }
    }
    wave_lds_fence();
    return true;
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
    const int x = wave_inclusive_scan(s);
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
    const int x = wave_inclusive_scan(s);
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
// Launch-side helpers shared by the schedules
// ----------------------------------------------------------------------------
// Vectors per lane in the permute row copy: up to 8 while a row has few
// copies (2-way fan-out measured best with full-row chunks), up to 4 for
// 4-way and wider fan-out (measured slightly faster: more waves in flight).
static constexpr int kCopyUnrolls[] = {8, 7, 6, 5, 4, 3, 2, 1};
static constexpr int kCopyUnrollsWideFanout[] = {4, 3, 2, 1};

// Row stores: plain stores when each row fans out to many destinations and
// the permuted output is large (measured faster for 8-way fan-out at 256 MiB
// and above); non-temporal otherwise (faster for 2-way fan-out and for small
// outputs).  Measured with buffer rotation well beyond the last-level cache.
static constexpr int kPlainStoreMinTopk = 4;
static constexpr int64_t kPlainStoreMinBytes = int64_t(32) << 20;

inline bool plain_row_stores(const PermuteArgs& a) {
    return a.topk >= kPlainStoreMinTopk && a.num_tokens * a.topk * a.row_vecs * 16 >= kPlainStoreMinBytes;
}

// Plain stores come with topk >= 4, whose row chunks are at most 4 vectors
// per lane (kCopyUnrollsWideFanout), so wider chunks are built for
// non-temporal stores only.
static constexpr int kPlainStoreMaxUnroll = kCopyUnrollsWideFanout[0];
static_assert(kPlainStoreMinTopk >= 4, "plain row stores only where the wide-fan-out chunk widths apply");

inline int map_entries(const PermuteArgs& a) { return a.expert_map != nullptr ? a.num_experts : 0; }

// The map and the id type are compile-time parameters of every permute
// kernel, so the plain int32 permute carries none of their code.  f receives
// std::integral_constant<bool, map> and a null `const IdT*` naming the id type.
template <class F>
inline void with_variant(const PermuteArgs& a, F&& f) {
    if (a.expert_map != nullptr) {
        if (a.ids64) f(std::true_type{}, static_cast<const int64_t*>(nullptr));
        else f(std::true_type{}, static_cast<const int32_t*>(nullptr));
    } else {
        if (a.ids64) f(std::false_type{}, static_cast<const int64_t*>(nullptr));
        else f(std::false_type{}, static_cast<const int32_t*>(nullptr));
    }
}

#define MOE_VARIANT_TYPES                                 \
    constexpr bool kMap = decltype(map_tag)::value;       \
    using IdT = std::remove_const_t<std::remove_pointer_t<decltype(id_tag)>>


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

}  // namespace moe
