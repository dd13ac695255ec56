// moe_gemm_kernels.hip -- grouped GEMM over the permuted rows (gfx950 MFMA).
//
// What is computed (vLLM PR #14568, "permute/unpermute kernel for moe
// optimization", PR description: a grouped GEMM runs the experts over the
// rows the permute made contiguous): for every expert e and every permuted row
// j in [off[e], off[e+1]),
//     y[j][n] = sum_k x[j][k] * w[e][n][k]
// with bf16 x and w, fp32 accumulation (MFMA), rounded once to bf16.
//
// Design:
//   * tiles of 128 rows x 128 output columns; a workgroup of 4 waves, each
//     wave a 64 x 64 quadrant of 2 x 2 v_mfma_f32_32x32x16_bf16 tiles; k
//     advances 64 at a time;
//   * both operands go from global memory straight into LDS (global_load_lds,
//     16 bytes per lane), 128-byte rows with the 16-byte k-vectors of row r
//     stored in slot (kvec ^ r % 8), so the fragment reads of 32 consecutive
//     rows hit every bank once; two LDS stages: while a step computes from one,
//     the next step's loads fill the other (one barrier per step);
//   * the tile list lives on the device: the offsets come from the permute, so
//     every workgroup derives the per-expert tile counts from them (prefix in
//     LDS) and walks tiles persistently.  Order: per expert, groups of 8 row
//     tiles, all column tiles of a group, row tiles fastest -- a group's rows
//     and a column tile's weights are reused while they are cached; the
//     concurrently running tiles are split into one contiguous chunk per XCD
//     (workgroups are dispatched round-robin over the 8 XCDs), so each XCD's
//     L2 sees neighbouring tiles.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;             // row tiles per group in the tile order
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct TileCoord {
    int expert;
    int64_t row0;   // first permuted row of the tile
    int64_t rows;   // rows of the tile that exist (<= BM)
    int64_t col0;   // first output column
};

// tile_pre[e] = tiles of experts < e (E + 1 entries in LDS).
template <int BM, int BN>
__device__ __forceinline__ TileCoord tile_coord(int64_t id, const int64_t* __restrict__ off, const int64_t* tile_pre,
                                                int num_experts, int64_t n_tiles) {
    int lo = 0, hi = num_experts - 1;  // last expert with tile_pre[e] <= id
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (tile_pre[mid] <= id) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int64_t local = id - tile_pre[e];
    const int64_t cnt = off[e + 1] - off[e];
    const int64_t mt = (cnt + BM - 1) / BM;
    const int64_t g = local / (kGroupM * n_tiles);
    const int64_t gsize = mt - g * kGroupM < kGroupM ? mt - g * kGroupM : kGroupM;
    const int64_t r = local - g * kGroupM * n_tiles;
    const int64_t nt = r / gsize;
    const int64_t mi = g * kGroupM + (r - nt * gsize);
    TileCoord c;
    c.expert = e;
    c.row0 = off[e] + mi * BM;
    c.rows = cnt - mi * BM < BM ? cnt - mi * BM : BM;
    c.col0 = nt * BN;
    return c;
}

// One k-step of one operand tile (ROWS rows x 64 bf16 = 128 bytes per row)
// loaded straight from global memory into LDS: wave w fills rows
// [w*ROWS/4, (w+1)*ROWS/4), one 1 KiB instruction (8 rows) at a time; lane L
// of an instruction writes slot L % 8 of row L / 8, and reads the row's
// k-vector (L % 8) ^ (row % 8) -- the XOR swizzle that keeps the fragment
// reads of 32 consecutive rows free of bank conflicts.
template <int ROWS>
__device__ __forceinline__ void tile_to_lds(__bf16* lds, const u32x4* __restrict__ src_row0, int64_t row_stride_vecs,
                                            int rows_valid, int64_t kvec0, int wave, int lane) {
    constexpr int kPerWave = ROWS / 4 / 8;  // instructions per wave
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        const int row = wave * (ROWS / 4) + j * 8 + lane / 8;
        const int slot = lane % 8;
        const int srow = row < rows_valid ? row : rows_valid - 1;  // clamp: a valid row, result unused
        const u32x4* g = src_row0 + (int64_t)srow * row_stride_vecs + kvec0 + (slot ^ (row % 8));
        __builtin_amdgcn_global_load_lds(g, lds + (wave * (ROWS / 4) + j * 8) * kBK, 16, 0, 0);
    }
}

// Fragment of 8 consecutive k (k-vector kvec) of tile row `row`.
__device__ __forceinline__ bf16x8 lds_frag(const __bf16* lds, int row, int kvec) {
    return *reinterpret_cast<const bf16x8*>(lds + row * kBK + ((kvec ^ (row % 8)) * 8));
}

// BM x BN output tile per workgroup of 4 waves (2 x 2), each wave
// (BM/2) x (BN/2) = MT x NT tiles of 32 x 32.  The MFMA takes the weight
// fragment as its first operand and the row fragment as its second, so a
// lane's 16 results are 4 runs of 4 consecutive output columns of one row
// (8-byte stores in the epilogue).
template <int BM, int BN>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n, int64_t k) {
    constexpr int MT = BM / 64, NT = BN / 64;  // 32 x 32 tiles per wave along m and n
    // Two stages per operand, each its own LDS object, so the compiler's wait
    // tracking can tell a stage being filled from the one being read.
    __shared__ __attribute__((aligned(1024))) __bf16 a_s0[BM * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 a_s1[BM * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 b_s0[BN * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 b_s1[BN * kBK];
    __shared__ int64_t tile_pre[kMaxExperts + 1];
    __shared__ int64_t part[kGemmThreads];
    __shared__ int bad_s;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = wave / 2, wn = wave % 2;  // this wave's quadrant
    const int64_t n_tiles = n / BN;
    const int64_t kv = k / 8;                // 16-byte vectors per row of x / w

    // The stages are written only by direct-to-LDS loads, which the compiler
    // does not see as stores: one visible store keeps their reads from being
    // folded away as reads of never-written memory.
    if (tid == 0) {
        a_s0[0] = a_s1[0] = b_s0[0] = b_s1[0] = (__bf16)0.0f;
    }

    // Tile counts per expert and their prefix (each thread takes kPer
    // consecutive experts; a scan over the threads in LDS), and a check of the
    // offsets (the permute writes -1 everywhere when it rejected an id).
    constexpr int kPer = (kMaxExperts + kGemmThreads - 1) / kGemmThreads;
    int64_t cnt_t[kPer];
    int64_t s = 0;
    int bad = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        cnt_t[q] = 0;
        if (e < num_experts) {
            const int64_t cnt = off[e + 1] - off[e];
            bad |= cnt < 0;
            cnt_t[q] = cnt > 0 ? (cnt + BM - 1) / BM * n_tiles : 0;
        }
        s += cnt_t[q];
    }
    if (tid == 0) bad |= off[0] != 0 || off[num_experts] > max_rows;
    if (tid == 0) bad_s = 0;
    part[tid] = s;
    __syncthreads();
    if (bad) atomicOr(&bad_s, 1);
    for (int d = 1; d < kGemmThreads; d <<= 1) {
        const int64_t v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t excl = part[tid] - s;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < num_experts) tile_pre[e] = excl;
        excl += cnt_t[q];
    }
    if (tid == 0) tile_pre[num_experts] = part[kGemmThreads - 1];
    __syncthreads();
    if (bad_s) return;
    const int64_t total = tile_pre[num_experts];

    // Persistent walk: iteration i covers tiles [i*G, (i+1)*G), G = gridDim.x;
    // XCD x (blocks b with b % 8 == x) takes the contiguous chunk x*G/8 ...
    const int64_t G = gridDim.x;
    const int64_t per_xcd = G / kXcds;
    const int64_t slot = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    for (int64_t base = 0; base < total; base += G) {
        const int64_t id = base + slot;
        if (id >= total) break;
        const TileCoord tc = tile_coord<BM, BN>(id, off, tile_pre, num_experts, n_tiles);
        const u32x4* xrow0 = x + tc.row0 * kv;
        const u32x4* wrow0 = w + ((int64_t)tc.expert * n + tc.col0) * kv;
        const int rows_valid = (int)tc.rows;

        f32x16 acc[MT][NT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x16{};

        auto load_step = [&](int64_t step, __bf16* as, __bf16* bs) {
            tile_to_lds<BM>(as, xrow0, kv, rows_valid, step * (kBK / 8), wave, lane);
            tile_to_lds<BN>(bs, wrow0, kv, BN, step * (kBK / 8), wave, lane);
        };
        auto compute_step = [&](const __bf16* as, const __bf16* bs) {
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                const int kvec = kk * 2 + lane / 32;
                bf16x8 af[MT], bfr[NT];
#pragma unroll
                for (int mi = 0; mi < MT; ++mi) af[mi] = lds_frag(as, wm * (BM / 2) + mi * 32 + lane % 32, kvec);
#pragma unroll
                for (int ni = 0; ni < NT; ++ni) bfr[ni] = lds_frag(bs, wn * (BN / 2) + ni * 32 + lane % 32, kvec);
#pragma unroll
                for (int mi = 0; mi < MT; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NT; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
            }
        };

        // Step ks computes from stage ks % 2 while step ks + 1 loads into the
        // other; one barrier per step (after it, step ks's data is visible and
        // every wave is done reading the stage that step ks + 1 overwrites).
        const int64_t ksteps = k / kBK;
        __syncthreads();  // the previous tile is done with both stages
        load_step(0, a_s0, b_s0);
        int64_t ks = 0;
        for (; ks + 1 < ksteps; ks += 2) {  // steps ks (stage 0) and ks + 1 (stage 1)
            __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of step ks have landed
            __syncthreads();
            load_step(ks + 1, a_s1, b_s1);
            compute_step(a_s0, b_s0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (ks + 2 < ksteps) load_step(ks + 2, a_s0, b_s0);
            compute_step(a_s1, b_s1);
        }
        if (ks < ksteps) {  // an odd last step, in stage 0
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            compute_step(a_s0, b_s0);
        }

        // Epilogue: for the 32 x 32 tile (weight rows n, x rows m), lane l,
        // register r holds n = (l / 32) * 4 + (r / 4) * 8 + r % 4, m = l % 32:
        // registers 4j .. 4j+3 are four consecutive output columns of row m.
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            const int row = wm * (BM / 2) + mi * 32 + lane % 32;
            if (row >= tc.rows) continue;
            uint16_t* yrow = y + (tc.row0 + row) * n;
#pragma unroll
            for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = tc.col0 + wn * (BN / 2) + ni * 32 + (lane / 32) * 4 + j * 8;
                    const uint32_t lo = bf16_bits_rne(acc[mi][ni][4 * j]) | (bf16_bits_rne(acc[mi][ni][4 * j + 1]) << 16);
                    const uint32_t hi =
                        bf16_bits_rne(acc[mi][ni][4 * j + 2]) | (bf16_bits_rne(acc[mi][ni][4 * j + 3]) << 16);
                    *reinterpret_cast<uint2*>(yrow + col) = make_uint2(lo, hi);
                }
            }
        }
    }
}

}  // namespace

namespace {

template <int BM, int BN>
hipError_t launch_gemm_tiles(const GemmArgs& a, int num_cus, int per_cu, hipStream_t stream) {
    // Persistent grid: per_cu workgroups per compute unit, a multiple of the XCD count.
    int64_t blocks = (int64_t)num_cus * per_cu;
    blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN>), dim3((unsigned)blocks), dim3(kGemmThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(a.x), reinterpret_cast<const u32x4*>(a.w), a.offsets,
                       reinterpret_cast<uint16_t*>(a.y), a.num_experts, a.max_rows, a.n, a.k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, int num_cus, hipStream_t stream) {
    return launch_gemm_tiles<128, 128>(a, num_cus, 2, stream);
}

}  // namespace moe
