// moe_plan.h -- host-side launch planning for the permute / unpermute kernels.
//
// Pure C++ with no HIP call, so the size query and the argument checks work on
// a host without a GPU.  The plan fixes, for one call:
//   * which permute schedule runs:
//       wave   -- one kernel of one-wave workgroups for at most kWaveMaxRows
//                 rows without an expert map (decode): every wave computes
//                 the whole index itself, with no workgroup barrier;
//       fused  -- one kernel; every workgroup counts all expert ids itself
//                 (cheap while N*topk is small, and it avoids extra launches);
//       coarse -- two kernels: expert counts per coarse tile (a few dozen),
//                 then the fused-style kernel whose counts outside its tile
//                 come from that histogram plus the rows that precede it in
//                 its coarse tile;
//       staged -- three kernels: per-tile stable ranks and histograms, a
//                 per-expert scan over tiles, then scatter + row copy (any
//                 size);
//   * how expanded rows are cut into tiles (whole tokens per tile);
//   * where each piece of the workspace lives.
// The sort runs over `buckets` keys: the experts, or with a local-expert map
// the local experts (rows of remote experts get no bucket).  `map_entries` is
// the length of that map (0 without one); the kernels stage it in LDS.
#pragma once

#include <cstddef>
#include <cstdint>
#include <initializer_list>

namespace moe {

constexpr int kWaveSize = 64;
constexpr int kFusedThreads = 512;                 // fused permute workgroup (8 waves)
constexpr int kRankThreads = 256;                  // staged kernel 1
constexpr int kScanThreads = 256;                  // staged kernel 2 (one workgroup per histogram row)
constexpr int kScatterThreads = 256;               // staged kernel 3
constexpr int kCoarseThreads = 512;                // coarse schedule, both kernels
constexpr int kCoarseMaxHist = 8192;               // coarse histogram entries held in LDS
constexpr int kCoarseMaxRowsPerTile = 8192;        // rows before a tile inside its coarse tile, at most
constexpr int kMaxCoarseTiles = 32;
constexpr int kMaxLdsInts = 16384;                 // 64 KiB of dynamic LDS per workgroup
constexpr int64_t kMaxGridBlocks = int64_t(1) << 20;  // beyond this, waves loop over further items
constexpr int kScanPerThread = 8;                  // tile counts one scan thread holds per pass
constexpr int kMaxExperts = 1024;
constexpr int64_t kFusedMaxRows = 16384;           // fused schedule up to this many expanded rows
constexpr int64_t kWaveMaxRows = 128;              // wave schedule up to this many rows (2 ids per lane)
constexpr int64_t kWaveMaxChunkBlocks = 4096;      // wave schedule grid (chunks per token); waves loop beyond
constexpr int kStagedTileRows = 128;               // target expanded rows per staged tile
constexpr int kCoarseCopyTileRows = 64;            // coarse tiles of a copying permute without an expert map
constexpr int kFusedTargetBlocks = 512;
constexpr int kMaxTileRows = 1024;                 // LDS staging bound for one tile
constexpr size_t kWorkspaceAlign = 256;
constexpr size_t kStaticScratchBytes = size_t(4) << 20;  // workspace of moe_permute_static_scratch
// Expanded-row bytes (N * topk * row bytes) from which a permute without an
// expert map takes the split schedule: the index-only schedule, then a
// separate row copy (moe_permute_rows.hip).  The index pass costs about
// 10 us at these sizes and the separate copy saves about 13 us per GB moved
// (DSv3 shape, 2.1 GB: 434 -> 416 us); the Qwen3 shape (0.3 GB) measured
// 58 -> 61 us with it.
constexpr int64_t kSplitCopyMinBytes = int64_t(1) << 30;
// With an expert map (a rank's share: about N * topk / ranks rows), from
// this many bytes of token rows (N * row bytes) at topk >= 4.  DSv3 shape,
// 8-way split: the three measured ranks' permutes 121 -> 115, 51 -> 46 and
// 56 -> 51 us; below it the index pass costs more than it saves (Qwen3 shape,
// 34 MB of token rows, 4- and 8-way: 25 -> 27 and 19 -> 21 us; Mixtral shape,
// topk 2, 2-way: 13 -> 20 us).
constexpr int64_t kSplitMapMinTokenBytes = int64_t(128) << 20;
constexpr int kSplitMapMinTopk = 4;
constexpr int kQuantMaxRowVecs = 1024;             // quantise-scatter: a wave holds the whole row (16 KiB)
constexpr int kIndexOnlyTileScale = 4;             // coarse tiles of an index-only permute, vs the staged ones

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Vectors per lane per work item (a chunk is U*64 16-byte vectors of one row).
// Picks the widest U from `allowed` (descending) whose chunks cover the row
// with at most 10% idle lanes, so rows split evenly (e.g. 14 groups of 64
// vectors -> U = 7, two full chunks).
inline int choose_unroll(int64_t row_vecs, const int* allowed, int n_allowed) {
    const int64_t groups = (row_vecs + kWaveSize - 1) / kWaveSize;
    if (groups <= 0) return allowed[n_allowed - 1];
    for (int i = 0; i < n_allowed; ++i) {
        const int64_t u = allowed[i];
        const int64_t lanes = (groups + u - 1) / u * u;
        if (groups * 10 >= lanes * 9) return (int)u;
    }
    return allowed[n_allowed - 1];
}

inline int key_bits(int buckets) {
    int b = 0;
    while ((1 << b) < buckets) ++b;
    return b;
}

struct PermutePlan {
    bool wave = false;            // one-wave workgroups, whole index per wave (no workspace)
    bool split_copy = false;      // index-only schedule below, then the separate row copy
    bool fused = false;
    bool coarse = false;          // two-kernel schedule (only when !fused)
    int coarse_rows = 0;          // expanded rows per coarse tile (a multiple of tile_rows)
    int num_coarse = 0;
    int64_t rows = 0;             // N * topk
    int tokens_per_tile = 1;
    int tile_rows = 0;            // tokens_per_tile * topk
    int64_t num_tiles = 0;
    int nbits = 0;
    // staged-schedule workspace layout (bytes from the workspace base)
    size_t ws_rank = 0;           // int32 [rows]           rank of each row within its tile
    size_t ws_tile_hist = 0;      // int32 [B+1][num_tiles] per-tile counts, then per-tile bases
    size_t ws_total = 0;          // int32 [B+1]            rows per bucket (+ bad-id count)
    size_t ws_bytes = 0;          // bytes this call needs
    // coarse schedule workspace: int32 [num_coarse][B+1] counts per coarse tile (+ bad ids)
    // (B = buckets: experts, or local experts with a map)
};

// Tokens per staged tile: about kStagedTileRows expanded rows, whole tokens.
inline int staged_tokens_per_tile(int topk) {
    int t = kStagedTileRows / topk;
    return t < 1 ? 1 : t;
}

// Tokens per coarse tile of a permute that copies rows and has no expert map:
// about kCoarseCopyTileRows rows.  Twice as many tiles as with staged-size
// tiles keeps more workgroups resident (four per CU instead of two at the
// Qwen3 shape, whose 512 staged-size tiles filled half the wave slots):
// Qwen3-shaped permute 63.0 -> 59.0 us; DSv3-shaped unchanged (write bound).
// With an expert map the staged size stays: a lightly loaded rank copies
// about one row per token, and its fixed per-tile index work then dominates
// (measured slower with 64-row tiles).
inline int coarse_copy_tokens_per_tile(int topk) {
    int t = kCoarseCopyTileRows / topk;
    return t < 1 ? 1 : t;
}

inline size_t staged_workspace_bytes(int64_t rows, int64_t num_tiles, int buckets) {
    size_t b = align_up(sizeof(int32_t) * (size_t)rows, kWorkspaceAlign);
    b += align_up(sizeof(int32_t) * (size_t)(buckets + 1) * (size_t)num_tiles, kWorkspaceAlign);
    b += align_up(sizeof(int32_t) * (size_t)(buckets + 1), kWorkspaceAlign);
    return b;
}

// Grid of the staged kernels: one workgroup per tile, as a 2-D grid so that
// num_tiles * threads never exceeds the 32-bit work-item count of one grid
// dimension (tiles of fewer than 128 rows, e.g. 126 for topk 3, reach it
// below the 2^31-row limit); workgroups past num_tiles return at once.
constexpr int64_t kStagedGridX = 65535;
inline void staged_grid(int64_t num_tiles, unsigned& gx, unsigned& gy) {
    const int64_t x = num_tiles < kStagedGridX ? (num_tiles > 0 ? num_tiles : 1) : kStagedGridX;
    gx = (unsigned)x;
    gy = (unsigned)((num_tiles + x - 1) / x > 0 ? (num_tiles + x - 1) / x : 1);
}

// Coarse tiles a problem may use: bounded by kMaxCoarseTiles, by the LDS held
// histogram (entries and the whole workgroup's LDS), for B buckets, a map of
// map_entries ints and tiles of tile_rows rows.
inline int max_coarse_tiles(int buckets, int tile_rows, int map_entries) {
    int n = kMaxCoarseTiles;
    const int by_hist = kCoarseMaxHist / (buckets + 1);
    const int by_lds =
        (kMaxLdsInts - 16 - map_entries - (1 + kCoarseThreads / kWaveSize) * buckets - tile_rows) / (buckets + 1);
    if (by_hist < n) n = by_hist;
    if (by_lds < n) n = by_lds;
    return n;
}

// Coarse tile length for R rows (a multiple of tile_rows), or 0 when the
// coarse schedule does not apply (too many rows per coarse tile).
inline int64_t coarse_rows_for(int64_t rows, int buckets, int tile_rows, int map_entries) {
    const int nmax = max_coarse_tiles(buckets, tile_rows, map_entries);
    if (nmax < 1) return 0;
    const int64_t per = (rows + nmax - 1) / nmax;
    const int64_t m = (per + tile_rows - 1) / tile_rows;
    const int64_t cr = m * tile_rows;
    return cr - tile_rows <= kCoarseMaxRowsPerTile ? cr : 0;
}

inline size_t coarse_workspace_bytes(int num_coarse, int buckets) {
    return align_up(sizeof(int32_t) * (size_t)num_coarse * (size_t)(buckets + 1), kWorkspaceAlign);
}

inline PermutePlan plan_permute(int64_t num_tokens, int topk, int buckets, int map_entries, bool index_only = false);

// Whether a permute copying rows of row_bytes takes the split schedule.
inline bool split_copy_applies(int64_t num_tokens, int topk, int64_t row_bytes, int map_entries) {
    if (row_bytes <= 0) return false;
    if (map_entries > 0) return topk >= kSplitMapMinTopk && num_tokens * row_bytes >= kSplitMapMinTokenBytes;
    return num_tokens * topk * row_bytes >= kSplitCopyMinBytes;
}

// Workspace of a call with max_num_tokens tokens; every call with fewer tokens
// needs no more.  A coarse call needs at most max_coarse_tiles histogram rows
// for the tile size it uses (the staged size, or the copy size without a map);
// a call takes the staged schedule only when the coarse one does not apply,
// which holds for every larger row count too, and the staged size grows with
// the row count -- so the plans at max_num_tokens bound the staged case.
inline size_t workspace_bound(int64_t max_num_tokens, int topk, int buckets, int map_entries) {
    const int64_t rows = max_num_tokens * topk;
    if (rows <= kFusedMaxRows) return 0;
    size_t b = 0;
    const int sizes[2] = {staged_tokens_per_tile(topk), coarse_copy_tokens_per_tile(topk)};
    for (int i = 0; i < (map_entries == 0 ? 2 : 1); ++i) {
        const int nmax = max_coarse_tiles(buckets, sizes[i] * topk, map_entries);
        if (nmax > 0 && coarse_workspace_bytes(nmax, buckets) > b) b = coarse_workspace_bytes(nmax, buckets);
    }
    for (bool index_only : {false, true}) {
        const size_t w = plan_permute(max_num_tokens, topk, buckets, map_entries, index_only).ws_bytes;
        if (w > b) b = w;
    }
    return b;
}

// index_only: no rows are copied (the quantising permute moves them in a
// second kernel), so fewer, larger tiles: every fused workgroup counts all ids,
// and without a row copy to hide behind that count is the kernel's cost.
inline PermutePlan plan_permute(int64_t num_tokens, int topk, int buckets, int map_entries, bool index_only) {
    PermutePlan p;
    p.rows = num_tokens * topk;
    p.nbits = key_bits(buckets);
    if (p.rows >= 1 && p.rows <= kWaveMaxRows && map_entries == 0) {
        p.wave = true;
        p.tokens_per_tile = (int)num_tokens;
        p.tile_rows = (int)p.rows;
        p.num_tiles = 1;
        return p;
    }
    if (p.rows <= kFusedMaxRows) {
        p.fused = true;
        // Enough workgroups to spread the row copy, at most kFusedThreads rows per tile.
        int64_t tpt = (num_tokens + kFusedTargetBlocks - 1) / kFusedTargetBlocks;
        const int64_t cap = (kFusedThreads / topk) < 1 ? 1 : (kFusedThreads / topk);
        if (tpt < 1) tpt = 1;
        if (index_only) tpt *= 8;
        if (tpt > cap) tpt = cap;
        p.tokens_per_tile = (int)tpt;
    } else {
        p.fused = false;
        p.tokens_per_tile = staged_tokens_per_tile(topk);
        const int small = coarse_copy_tokens_per_tile(topk);
        if (!index_only && map_entries == 0 && small < p.tokens_per_tile &&
            coarse_rows_for(p.rows, buckets, small * topk, map_entries) > 0)
            p.tokens_per_tile = small;
    }
    if (!p.fused && index_only) {
        // Without a row copy the fixed index work of each tile is the cost, so
        // the coarse schedule takes tiles kIndexOnlyTileScale times the staged
        // size (whole tokens, at most kMaxTileRows rows) where it still applies
        // with them; the histogram then has no more rows than with the
        // staged-size tiles, so the workspace bound holds.
        int64_t big = (int64_t)p.tokens_per_tile * kIndexOnlyTileScale;
        const int64_t cap = kMaxTileRows / topk;
        if (big > cap) big = cap;
        if (big > p.tokens_per_tile && coarse_rows_for(p.rows, buckets, (int)(big * topk), map_entries) > 0)
            p.tokens_per_tile = (int)big;
    }
    p.tile_rows = p.tokens_per_tile * topk;
    p.num_tiles = num_tokens == 0 ? 0 : (num_tokens + p.tokens_per_tile - 1) / p.tokens_per_tile;
    if (!p.fused) {
        const int64_t cr = coarse_rows_for(p.rows, buckets, p.tile_rows, map_entries);
        if (cr > 0) {
            p.coarse = true;
            p.coarse_rows = (int)cr;
            p.num_coarse = (int)((p.rows + cr - 1) / cr);
            p.ws_bytes = coarse_workspace_bytes(p.num_coarse, buckets);
        } else {
            p.ws_rank = 0;
            p.ws_tile_hist = align_up(sizeof(int32_t) * (size_t)p.rows, kWorkspaceAlign);
            p.ws_total = p.ws_tile_hist +
                         align_up(sizeof(int32_t) * (size_t)(buckets + 1) * (size_t)p.num_tiles, kWorkspaceAlign);
            p.ws_bytes = staged_workspace_bytes(p.rows, p.num_tiles, buckets);
        }
    }
    return p;
}

// Dynamic LDS bytes of each kernel for one tile shape (B buckets; the map,
// when there is one, sits after everything else).
inline size_t wave_lds_bytes(int experts, int rows) { return sizeof(int) * ((size_t)experts + (size_t)rows); }
inline size_t fused_lds_bytes(int buckets, int tile_rows, int map_entries) {
    return sizeof(int) *
           ((size_t)(2 + kFusedThreads / kWaveSize) * buckets + (size_t)tile_rows + 16 + (size_t)map_entries);
}
inline size_t rank_lds_bytes(int buckets, int tile_rows, int map_entries) {
    return sizeof(int) *
           ((size_t)(1 + kRankThreads / kWaveSize) * buckets + 2 * (size_t)tile_rows + 16 + (size_t)map_entries);
}
inline size_t coarse_hist_lds_bytes(int buckets, int map_entries) {
    return sizeof(int) * ((size_t)(buckets + 1) + (size_t)map_entries);
}
inline size_t coarse_scatter_lds_bytes(int buckets, int tile_rows, int num_coarse, int map_entries) {
    return sizeof(int) * ((size_t)num_coarse * (buckets + 1) + (size_t)(1 + kCoarseThreads / kWaveSize) * buckets +
                          (size_t)tile_rows + 16 + (size_t)map_entries);
}
inline size_t scatter_lds_bytes(int buckets, int tile_rows, int map_entries) {
    return sizeof(int) * ((size_t)(2 * buckets + 1) + (size_t)tile_rows + 16 + (size_t)map_entries);
}

}  // namespace moe
