// moe_gemm_kernels.hip -- grouped GEMM over the permuted rows (gfx950 MFMA).
//
// What is computed (vLLM PR #14568, "permute/unpermute kernel for moe
// optimization", PR description: a grouped GEMM runs the experts over the
// rows the permute made contiguous): for every expert e and every permuted row
// j in [off[e], off[e+1]),
//     y[j][n] = sum_k x[j][k] * w[e][n][k]
// with bf16 x and w, fp32 accumulation (MFMA), rounded once to bf16.
//
// Design (a first MFMA version):
//   * tiles of 128 rows x 128 output columns; a workgroup of 4 waves, each wave
//     64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16 tiles; k advances 64 at a time;
//   * both operands are "row, 8 consecutive k" fragments, staged in LDS with a
//     row pitch of 72 elements (144 bytes) so the 16-byte fragment reads of 32
//     consecutive rows fall in different banks; the next k-step's global loads
//     are issued into registers before the current step's MFMAs;
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

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kPitch = kBK + 8;        // LDS row pitch in bf16 elements (144 bytes)
constexpr int kGroupM = 8;             // row tiles per group in the tile order
constexpr int kXcds = 8;
constexpr int kTileVecs = kBM * kBK / 8;                  // 16-byte vectors per operand tile (1024)
constexpr int kVecsPerThread = kTileVecs / kGemmThreads;  // 4

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct TileCoord {
    int expert;
    int64_t row0;   // first permuted row of the tile
    int64_t rows;   // rows of the tile that exist (<= kBM)
    int64_t col0;   // first output column
};

// tile_pre[e] = tiles of experts < e (E + 1 entries in LDS).
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
    const int64_t mt = (cnt + kBM - 1) / kBM;
    const int64_t g = local / (kGroupM * n_tiles);
    const int64_t gsize = mt - g * kGroupM < kGroupM ? mt - g * kGroupM : kGroupM;
    const int64_t r = local - g * kGroupM * n_tiles;
    const int64_t nt = r / gsize;
    const int64_t mi = g * kGroupM + (r - nt * gsize);
    TileCoord c;
    c.expert = e;
    c.row0 = off[e] + mi * kBM;
    c.rows = cnt - mi * kBM < kBM ? cnt - mi * kBM : kBM;
    c.col0 = nt * kBN;
    return c;
}

__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n, int64_t k) {
    __shared__ __attribute__((aligned(16))) __bf16 a_s[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) __bf16 b_s[kBN * kPitch];
    __shared__ int64_t tile_pre[kMaxExperts + 1];
    __shared__ int64_t part[kGemmThreads];
    __shared__ int bad_s;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = tid / 64;
    const int wm = wave / 2, wn = wave % 2;  // this wave's 64 x 64 quadrant
    const int64_t n_tiles = n / kBN;
    const int64_t kv = k / 8;                // 16-byte vectors per row of x / w

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
            cnt_t[q] = cnt > 0 ? (cnt + kBM - 1) / kBM * n_tiles : 0;
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
        const TileCoord tc = tile_coord(id, off, tile_pre, num_experts, n_tiles);
        const u32x4* wexp = w + (int64_t)tc.expert * n * kv;

        // This thread's share of each k-step: 4 vectors of the A tile and 4 of
        // the B tile (row = v / 8, k-vector = v % 8, v = tid + 256 i).
        int64_t a_src[kVecsPerThread], b_src[kVecsPerThread];
#pragma unroll
        for (int i = 0; i < kVecsPerThread; ++i) {
            const int v = tid + kGemmThreads * i;
            const int row = v / 8, kvec = v % 8;
            const int64_t arow = tc.row0 + (row < tc.rows ? row : tc.rows - 1);  // clamp: a valid row, result unused
            a_src[i] = arow * kv + kvec;
            b_src[i] = (tc.col0 + row) * kv + kvec;
        }
        u32x4 a_reg[kVecsPerThread], b_reg[kVecsPerThread];
#pragma unroll
        for (int i = 0; i < kVecsPerThread; ++i) {
            a_reg[i] = x[a_src[i]];  // plain loads: rows are reused across column tiles,
            b_reg[i] = wexp[b_src[i]];  // weights across row tiles
        }

        f32x16 acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

        const int64_t ksteps = k / kBK;
        for (int64_t ks = 0; ks < ksteps; ++ks) {
            __syncthreads();  // the previous step's fragment reads are done
#pragma unroll
            for (int i = 0; i < kVecsPerThread; ++i) {
                const int v = tid + kGemmThreads * i;
                const int row = v / 8, kvec = v % 8;
                *reinterpret_cast<u32x4*>(&a_s[row * kPitch + kvec * 8]) = a_reg[i];
                *reinterpret_cast<u32x4*>(&b_s[row * kPitch + kvec * 8]) = b_reg[i];
            }
            __syncthreads();
            if (ks + 1 < ksteps) {  // next step's loads fly while this step computes
                const int64_t koff = (ks + 1) * (kBK / 8);
#pragma unroll
                for (int i = 0; i < kVecsPerThread; ++i) {
                    a_reg[i] = x[a_src[i] + koff];
                    b_reg[i] = wexp[b_src[i] + koff];
                }
            }
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                const int kcol = kk * 16 + (lane / 32) * 8;
                bf16x8 af[2], bfr[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    af[mi] = *reinterpret_cast<const bf16x8*>(&a_s[(wm * 64 + mi * 32 + lane % 32) * kPitch + kcol]);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    bfr[ni] = *reinterpret_cast<const bf16x8*>(&b_s[(wn * 64 + ni * 32 + lane % 32) * kPitch + kcol]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
            }
        }

        // Epilogue: lane l, register r of a 32 x 32 tile holds
        // row (l / 32) * 4 + (r / 4) * 8 + r % 4, column l % 32.
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int64_t col = tc.col0 + wn * 64 + ni * 32 + lane % 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * 64 + mi * 32 + (lane / 32) * 4 + (r / 4) * 8 + r % 4;
                    if (row < tc.rows) y[(tc.row0 + row) * n + col] = (uint16_t)bf16_bits_rne(acc[mi][ni][r]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, int num_cus, hipStream_t stream) {
    // Persistent grid: two workgroups per compute unit, a multiple of the XCD count.
    int64_t blocks = (int64_t)num_cus * 2;
    blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel, dim3((unsigned)blocks), dim3(kGemmThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(a.x), reinterpret_cast<const u32x4*>(a.w), a.offsets,
                       reinterpret_cast<uint16_t*>(a.y), a.num_experts, a.max_rows, a.n, a.k);
    return hipGetLastError();
}

}  // namespace moe
