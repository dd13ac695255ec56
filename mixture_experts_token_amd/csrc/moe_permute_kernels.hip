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
// topk destinations, so HBM reads equal the algorithmic N*H bytes.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// Wavefront helpers
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

// Exclusive prefix sum of data[0..n) in LDS, in place; returns the total.
// Every thread of the workgroup must call it.  tmp: kBlockWaves ints of LDS.
__device__ int block_exclusive_scan(int* data, int n, int* tmp) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid % kWaveSize, w = tid / kWaveSize;
    const int per = (n + nt - 1) / nt;
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
    __syncthreads();
    int before = 0, total = 0;
    for (int v = 0; v < nt / kWaveSize; ++v) {
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
    __syncthreads();
    return total;
}

// ----------------------------------------------------------------------------
// Stable ranks within one tile of expanded rows [row0, row0 + tile_rows).
//
// Wave w owns rows [w*span, (w+1)*span) of the tile and walks them 64 at a
// time, so a row's rank is (rows of its expert in earlier waves) + (rows of
// its expert earlier in its own wave).  On return, after a barrier:
//   key_s[i]  expert of tile row i, or -1 if its id is out of range
//   rank_s[i] rank of row i among the tile's rows with the same expert
//   cnt_s[e]  rows of the tile routed to expert e
//   *bad_s    incremented by the tile's rows with an out-of-range id
// wave_s (kBlockWaves * E ints) must be zero on entry; it is clobbered.
// ----------------------------------------------------------------------------
__device__ void rank_tile(const int32_t* __restrict__ ids, int64_t row0, int tile_rows, int E, int nbits,
                          int* key_s, int* rank_s, int* wave_s, int* cnt_s, int* bad_s) {
    const int w = wave_index();
    const int lane = threadIdx.x % kWaveSize;
    const int span = (tile_rows + kBlockThreads - 1) / kBlockThreads * kWaveSize;
    const int beg = w * span;
    const int end = min(beg + span, tile_rows);
    int* run = wave_s + w * E;
    int nbad = 0;
    for (int base = beg; base < end; base += kWaveSize) {
        const int i = base + lane;
        const bool in_tile = i < end;
        const int key = in_tile ? ids[row0 + i] : 0;
        const bool ok = in_tile && (unsigned)key < (unsigned)E;
        nbad += (in_tile && !ok) ? 1 : 0;
        const uint64_t same = lanes_with_same_key(key, ok, nbits);
        const int below = lanes_below(same);
        if (ok) {
            const int r = run[key];
            rank_s[i] = r + below;
            key_s[i] = key;
            if (below == 0) run[key] = r + (int)__popcll(same);
        } else if (in_tile) {
            key_s[i] = -1;
            rank_s[i] = 0;
        }
    }
    if (nbad) atomicAdd(bad_s, nbad);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int s = 0;
        for (int v = 0; v < kBlockWaves; ++v) {
            const int c = wave_s[v * E + e];
            wave_s[v * E + e] = s;
            s += c;
        }
        cnt_s[e] = s;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < tile_rows; i += blockDim.x) {
        const int key = key_s[i];
        if (key >= 0) rank_s[i] += wave_s[(i / span) * E + key];
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// Row copy of one tile: token-major, each token row read once and written to
// its topk destinations.  Work items are (token, chunk of U*64 16-byte
// vectors); waves take items round-robin.  dest_s[tl*topk + k] is the
// permuted row of the tile's token tl, slot k.
// ----------------------------------------------------------------------------
template <int U>
__device__ __forceinline__ void copy_tile_rows(const PermuteArgs& a, int64_t t0, int ntok, const int* dest_s) {
    const int w = wave_index();
    const int lane = threadIdx.x % kWaveSize;
    const int K = a.topk;
    const int64_t rows_total = a.num_tokens * K;
    if (a.row_vecs > 0) {
        const int64_t rv = a.row_vecs;
        const int chunk = U * kWaveSize;
        const int nchunks = (int)((rv + chunk - 1) / chunk);
        const int items = ntok * nchunks;
        const u32x4* __restrict__ src_base = reinterpret_cast<const u32x4*>(a.hidden_states);
        u32x4* __restrict__ dst_base = reinterpret_cast<u32x4*>(a.permuted_hidden_states);
        for (int it = w; it < items; it += kBlockWaves) {
            const int tl = it / nchunks;
            const int c = it - tl * nchunks;
            const u32x4* src = src_base + (t0 + tl) * rv;
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = (int64_t)c * chunk + u * kWaveSize + lane;
                if (idx < rv) v[u] = __builtin_nontemporal_load(src + idx);
            }
            for (int k = 0; k < K; ++k) {
                const int d = dest_s[tl * K + k];
                if ((uint32_t)d >= (uint64_t)rows_total) continue;  // never taken when the ranks are right
                u32x4* dst = dst_base + (int64_t)d * rv;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t idx = (int64_t)c * chunk + u * kWaveSize + lane;
                    if (idx < rv) __builtin_nontemporal_store(v[u], dst + idx);
                }
            }
        }
    }
    if (a.token_scale != nullptr) {
        const int rows = ntok * K;
        for (int i = threadIdx.x; i < rows; i += blockDim.x) {
            const int d = dest_s[i];
            if ((uint32_t)d < (uint64_t)rows_total) a.permuted_scale[d] = a.token_scale[t0 + i / K];
        }
    }
}

// ----------------------------------------------------------------------------
// Fused permute: one workgroup per tile of whole tokens.  Every workgroup
// counts the expert ids of all rows outside its tile (before / after it),
// ranks its own rows, derives expert_first_token_offset and its own base per
// expert, scatters permuted_idx / inv_permuted_idx and copies its rows.
// ----------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kBlockThreads) void permute_fused_kernel(PermuteArgs a, int tokens_per_tile,
                                                                      int nbits) {
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int K = a.topk;
    const int64_t t0 = (int64_t)blockIdx.x * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int64_t row0 = t0 * K;
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;
    const int64_t R = a.num_tokens * K;

    int* before_s = smem;                       // [E] rows before the tile, then the tile's base
    int* after_s = before_s + E;                // [E] rows after the tile, then offsets
    int* cnt_s = after_s + E;                   // [E] rows inside the tile
    int* wave_s = cnt_s + E;                    // [kBlockWaves * E]
    int* key_s = wave_s + kBlockWaves * E;      // [tile_cap]
    int* rank_s = key_s + tile_cap;             // [tile_cap] rank, then destination
    int* misc_s = rank_s + tile_cap;            // [16]: [0] bad ids, [1..] scan scratch

    for (int i = threadIdx.x; i < (3 + kBlockWaves) * E; i += blockDim.x) smem[i] = 0;
    if (threadIdx.x < 16) misc_s[threadIdx.x] = 0;
    __syncthreads();

    int nbad = 0;
    for (int64_t r = threadIdx.x; r < R; r += blockDim.x) {
        if (r >= row0 && r < row0 + T) continue;
        const int key = a.topk_ids[r];
        if ((unsigned)key >= (unsigned)E) {
            ++nbad;
            continue;
        }
        atomicAdd(r < row0 ? &before_s[key] : &after_s[key], 1);
    }
    if (nbad) atomicAdd(&misc_s[0], nbad);

    rank_tile(a.topk_ids, row0, T, E, nbits, key_s, rank_s, wave_s, cnt_s, &misc_s[0]);

    if (misc_s[0] != 0) {  // every workgroup saw every id, so all take this branch together
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e <= E; e += blockDim.x) a.expert_first_token_offset[e] = -1;
        return;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) after_s[e] += before_s[e] + cnt_s[e];
    __syncthreads();
    const int total = block_exclusive_scan(after_s, E, misc_s + 1);
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e < E; e += blockDim.x) a.expert_first_token_offset[e] = after_s[e];
        if (threadIdx.x == 0) a.expert_first_token_offset[E] = total;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) before_s[e] += after_s[e];
    __syncthreads();
    for (int i = threadIdx.x; i < T; i += blockDim.x) {
        const int dest = before_s[key_s[i]] + rank_s[i];
        rank_s[i] = dest;
        a.inv_permuted_idx[row0 + i] = dest;
        if ((uint32_t)dest < (uint64_t)R) a.permuted_idx[dest] = (int32_t)(row0 + i);
    }
    __syncthreads();
    copy_tile_rows<U>(a, t0, ntok, rank_s);
}

// ----------------------------------------------------------------------------
// Staged permute, kernel 1: per tile, stable ranks and the expert histogram.
// rank_ws[r] = rank of row r within its tile; tile_hist[e][tile] = count,
// tile_hist[E][tile] = rows with an out-of-range id.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void permute_rank_tiles_kernel(PermuteArgs a, int tokens_per_tile,
                                                                           int nbits, int64_t num_tiles,
                                                                           int32_t* rank_ws, int32_t* tile_hist) {
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int K = a.topk;
    const int64_t tile = blockIdx.x;
    const int64_t t0 = tile * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int64_t row0 = t0 * K;
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;

    int* cnt_s = smem;                          // [E]
    int* wave_s = cnt_s + E;                    // [kBlockWaves * E]
    int* key_s = wave_s + kBlockWaves * E;      // [tile_cap]
    int* rank_s = key_s + tile_cap;             // [tile_cap]
    int* misc_s = rank_s + tile_cap;            // [16]

    for (int i = threadIdx.x; i < (1 + kBlockWaves) * E; i += blockDim.x) smem[i] = 0;
    if (threadIdx.x < 16) misc_s[threadIdx.x] = 0;
    __syncthreads();
    rank_tile(a.topk_ids, row0, T, E, nbits, key_s, rank_s, wave_s, cnt_s, &misc_s[0]);
    for (int i = threadIdx.x; i < T; i += blockDim.x) rank_ws[row0 + i] = rank_s[i];
    for (int e = threadIdx.x; e < E; e += blockDim.x) tile_hist[(int64_t)e * num_tiles + tile] = cnt_s[e];
    if (threadIdx.x == 0) tile_hist[(int64_t)E * num_tiles + tile] = misc_s[0];
}

// ----------------------------------------------------------------------------
// Staged permute, kernel 2: one wave per histogram row (expert, or the
// bad-id row E).  Exclusive scan over tiles in place, row total to total[e].
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void permute_scan_tiles_kernel(int32_t* tile_hist, int64_t num_tiles,
                                                                           int num_rows_hist, int32_t* total) {
    const int lane = threadIdx.x % kWaveSize;
    const int e = blockIdx.x * kBlockWaves + wave_index();
    if (e >= num_rows_hist) return;
    int32_t* row = tile_hist + (int64_t)e * num_tiles;
    int carry = 0;
    for (int64_t base = 0; base < num_tiles; base += kWaveSize) {
        const int64_t i = base + lane;
        const int v = i < num_tiles ? row[i] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < kWaveSize; d <<= 1) {
            const int y = __shfl_up(x, d, kWaveSize);
            if (lane >= d) x += y;
        }
        if (i < num_tiles) row[i] = carry + x - v;
        carry += __shfl(x, kWaveSize - 1, kWaveSize);
    }
    if (lane == 0) total[e] = carry;
}

// ----------------------------------------------------------------------------
// Staged permute, kernel 3: offsets from the per-expert totals, destinations
// from offset + tile base + rank, index scatter, and the row copy.
// ----------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kBlockThreads) void permute_scatter_kernel(PermuteArgs a, int tokens_per_tile,
                                                                        int64_t num_tiles, const int32_t* rank_ws,
                                                                        const int32_t* tile_base,
                                                                        const int32_t* total) {
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int K = a.topk;
    const int64_t tile = blockIdx.x;
    const int64_t t0 = tile * tokens_per_tile;
    const int ntok = (int)min((int64_t)tokens_per_tile, a.num_tokens - t0);
    const int64_t row0 = t0 * K;
    const int T = ntok * K;
    const int tile_cap = tokens_per_tile * K;

    int* off_s = smem;                // [E + 1]
    int* dest_s = off_s + (E + 1);    // [tile_cap]
    int* misc_s = dest_s + tile_cap;  // [16]

    for (int e = threadIdx.x; e < E; e += blockDim.x) off_s[e] = total[e];
    __syncthreads();
    if (total[E] != 0) {  // some id was out of range: report through the offsets, write nothing else
        if (tile == 0)
            for (int e = threadIdx.x; e <= E; e += blockDim.x) a.expert_first_token_offset[e] = -1;
        return;
    }
    const int rows_total = block_exclusive_scan(off_s, E, misc_s);
    if (tile == 0) {
        for (int e = threadIdx.x; e < E; e += blockDim.x) a.expert_first_token_offset[e] = off_s[e];
        if (threadIdx.x == 0) a.expert_first_token_offset[E] = rows_total;
    }
    const int64_t R = a.num_tokens * K;
    for (int i = threadIdx.x; i < T; i += blockDim.x) {
        const int64_t r = row0 + i;
        const int key = min(max(a.topk_ids[r], 0), E - 1);  // all ids are in range here (total[E] == 0)
        const int dest = off_s[key] + tile_base[(int64_t)key * num_tiles + tile] + rank_ws[r];
        dest_s[i] = dest;
        a.inv_permuted_idx[r] = dest;
        if ((uint32_t)dest < (uint64_t)R) a.permuted_idx[dest] = (int32_t)r;
    }
    __syncthreads();
    copy_tile_rows<U>(a, t0, ntok, dest_s);
}

__global__ void fill_offsets_kernel(int64_t* off, int n, int64_t value) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) off[i] = value;
}

// ----------------------------------------------------------------------------
// Unpermute: one wave per (token, chunk of U*64 16-byte vectors).  The topk
// rows of the token are read, weighted and summed in fp32 in ascending k,
// then rounded once to the element type.
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
__global__ __launch_bounds__(kBlockThreads) void unpermute_kernel(UnpermuteArgs a) {
    constexpr int kEl = kBF16 ? 8 : 4;  // elements per 16-byte vector
    const int lane = threadIdx.x % kWaveSize;
    const int64_t rv = a.row_vecs;
    const int chunk = U * kWaveSize;
    const int64_t nchunks = (rv + chunk - 1) / chunk;
    const int64_t item = (int64_t)blockIdx.x * kBlockWaves + wave_index();
    if (item >= a.num_tokens * nchunks) return;
    const int64_t t = item / nchunks;
    const int64_t c = item - t * nchunks;
    const int K = a.topk;
    const int64_t R = a.num_tokens * K;
    const u32x4* __restrict__ y = reinterpret_cast<const u32x4*>(a.expanded_output);

    float acc[U][kEl];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kEl; ++e) acc[u][e] = 0.0f;
    bool bad = false;
    for (int k = 0; k < K; ++k) {
        const int32_t j = a.inv_permuted_idx[t * K + k];
        const float wk = a.topk_weights[t * K + k];
        if (j < 0 || (int64_t)j >= R) {
            bad = true;
            continue;
        }
        const u32x4* src = y + (int64_t)j * rv;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = c * chunk + u * kWaveSize + lane;
            v[u] = idx < rv ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
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
    u32x4* __restrict__ out = reinterpret_cast<u32x4*>(a.output) + t * rv;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t idx = c * chunk + u * kWaveSize + lane;
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

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------
static constexpr int kCopyUnroll = 4;
static constexpr int kUnpermuteUnroll = 4;

hipError_t launch_fill_offsets(int64_t* off, int num_experts, int64_t value, hipStream_t stream) {
    hipLaunchKernelGGL(fill_offsets_kernel, dim3(1), dim3(kBlockThreads), 0, stream, off, num_experts + 1, value);
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t stream) {
    const int E = a.num_experts;
    if (p.fused) {
        const size_t lds = fused_lds_bytes(E, p.tile_rows);
        hipLaunchKernelGGL(permute_fused_kernel<kCopyUnroll>, dim3((unsigned)p.num_tiles), dim3(kBlockThreads),
                           lds, stream, a, p.tokens_per_tile, p.nbits);
        return hipGetLastError();
    }
    char* ws = static_cast<char*>(workspace);
    int32_t* rank_ws = reinterpret_cast<int32_t*>(ws + p.ws_rank);
    int32_t* tile_hist = reinterpret_cast<int32_t*>(ws + p.ws_tile_hist);
    int32_t* total = reinterpret_cast<int32_t*>(ws + p.ws_total);
    hipLaunchKernelGGL(permute_rank_tiles_kernel, dim3((unsigned)p.num_tiles), dim3(kBlockThreads),
                       rank_lds_bytes(E, p.tile_rows), stream, a, p.tokens_per_tile, p.nbits, p.num_tiles, rank_ws,
                       tile_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int hist_rows = E + 1;
    hipLaunchKernelGGL(permute_scan_tiles_kernel, dim3((unsigned)((hist_rows + kBlockWaves - 1) / kBlockWaves)),
                       dim3(kBlockThreads), 0, stream, tile_hist, p.num_tiles, hist_rows, total);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scatter_kernel<kCopyUnroll>, dim3((unsigned)p.num_tiles), dim3(kBlockThreads),
                       scatter_lds_bytes(E, p.tile_rows), stream, a, p.tokens_per_tile, p.num_tiles, rank_ws,
                       tile_hist, total);
    return hipGetLastError();
}

hipError_t launch_unpermute(const UnpermuteArgs& a, bool bf16, hipStream_t stream) {
    const int64_t chunk = kUnpermuteUnroll * kWaveSize;
    const int64_t nchunks = (a.row_vecs + chunk - 1) / chunk;
    const int64_t items = a.num_tokens * nchunks;
    const int64_t blocks = (items + kBlockWaves - 1) / kBlockWaves;
    if (bf16)
        hipLaunchKernelGGL((unpermute_kernel<true, kUnpermuteUnroll>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((unpermute_kernel<false, kUnpermuteUnroll>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace moe
