// moe_gemm_skinny.hip -- grouped GEMM for experts with few rows each (decode).
//
// What is computed is the grouped GEMM of moe_gemm_kernels.hip (vLLM PR
// #14568, PR description: a grouped GEMM over the rows the permute made
// contiguous): y[j][c] = sum_i x[j][i] * w[e][c][i] for the permuted rows j of
// expert e, bf16 in, fp32 accumulation, rounded once to bf16.
//
// At decode sizes an expert has one to a few dozen rows, so the work is
// streaming the experts' weights (n x k each) once: the bound is HBM, not the
// matrix cores.  The tiled kernel stages both operands through LDS in
// 128 x 256 tiles, which for a handful of rows leaves few tiles (one expert
// row of 256 columns each) and two or three k-steps of weight loads in flight
// per CU.  Here one wave owns 32 weight rows (output columns) of one expert
// and up to 16 of its x rows, streams those weight rows straight from global
// memory into MFMA operand registers (no LDS, no barrier) and keeps kSkDepth
// 64-wide k chunks of loads in flight.  The x fragments of a chunk are loaded
// with its weight fragments, so loads are consumed in issue order (the
// vector-memory counter retires in order).  Experts with more than 16 rows
// take several row groups, each streaming the weight rows again.
//
// MFMA operands (v_mfma_f32_16x16x32_bf16, weight fragment first): for the
// k half h (32 k) of a chunk, lane l holds 8 consecutive k (k-vector
// 4h + l / 16 of the chunk) of weight row l % 16 of a 16-row block and of x
// row l % 16, so the four lanes of a row read 64 contiguous bytes; lane l's
// 4 results are x row l % 16, output columns 4 (l / 16) .. 4 (l / 16) + 3 of
// the block.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kSkCols = 32;   // weight rows (output columns) per wave: two 16-row MFMA blocks
constexpr int kSkRows = 16;   // x rows per wave (one row group)
constexpr int kSkDepth = 4;   // 64-wide k chunks in flight per wave
constexpr int kSkThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The weight fragments (2 blocks x 2 k halves) and x fragments (2 k halves)
// of one 64-wide k chunk (k-vectors 8c .. 8c+7 of each row).
struct Chunk {
    u32x4 w[2][2];
    u32x4 x[2];
};

// wrow: this lane's row of weight block 0 (block 1 is 16 rows further on);
// q = lane / 16 picks the k-vector within a 32-wide half.
__device__ __forceinline__ void load_chunk(Chunk& ch, const u32x4* __restrict__ wrow, int64_t block_stride,
                                           const u32x4* __restrict__ xrow, int64_t c, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < 2; ++b) ch.w[b][h] = __builtin_nontemporal_load(wrow + b * block_stride + c * 8 + 4 * h + q);
        ch.x[h] = xrow[c * 8 + 4 * h + q];
    }
}

__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[2], const Chunk& ch) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ch.w[b][h]),
                                                             __builtin_bit_cast(bf16x8, ch.x[h]), acc[b], 0, 0, 0);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Work item = (expert, row group of 16 rows, block of 32 output columns);
// items of one expert are row-group major, so the column blocks of a row
// group run on neighbouring waves (one CU) and share its x rows in cache.
__global__ __launch_bounds__(kSkThreads) void grouped_gemm_skinny_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n, int64_t k) {
    __shared__ int64_t item_pre[kMaxExperts + 1];
    __shared__ int64_t part[kSkThreads];
    __shared__ int bad_s;
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int64_t nblocks = n / kSkCols;
    const int64_t kv = k / 8;  // 16-byte vectors per row
    const int64_t nchunks = k / 64;

    // Items per expert and their prefix; the offsets are checked as in the
    // tiled kernel (the permute writes -1 everywhere when it rejected an id).
    constexpr int kPer = (kMaxExperts + kSkThreads - 1) / kSkThreads;
    int64_t cnt_t[kPer];
    int64_t sum = 0;
    int bad = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        cnt_t[q] = 0;
        if (e < num_experts) {
            const int64_t cnt = off[e + 1] - off[e];
            bad |= cnt < 0;
            cnt_t[q] = cnt > 0 ? (cnt + kSkRows - 1) / kSkRows * nblocks : 0;
        }
        sum += cnt_t[q];
    }
    if (tid == 0) bad |= off[0] != 0 || off[num_experts] > max_rows;
    if (tid == 0) bad_s = 0;
    part[tid] = sum;
    __syncthreads();
    if (bad) atomicOr(&bad_s, 1);
    for (int d = 1; d < kSkThreads; d <<= 1) {
        const int64_t v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t excl = part[tid] - sum;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < num_experts) item_pre[e] = excl;
        excl += cnt_t[q];
    }
    if (tid == 0) item_pre[num_experts] = part[kSkThreads - 1];
    __syncthreads();
    if (bad_s) return;
    const int64_t total = item_pre[num_experts];
    const int64_t total_waves = (int64_t)gridDim.x * (kSkThreads / 64);

    for (int64_t id = (int64_t)blockIdx.x * (kSkThreads / 64) + wave; id < total; id += total_waves) {
        int lo = 0, hi = num_experts - 1;  // last expert with item_pre[e] <= id
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (item_pre[mid] <= id) lo = mid;
            else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int64_t local = id - item_pre[e];
        const int64_t group = local / nblocks;
        const int64_t col0 = uniform64((local - group * nblocks) * kSkCols);
        const int64_t row0 = uniform64(off[e] + group * kSkRows);
        const int64_t cnt = off[e + 1] - off[e];
        const int rows = (int)uniform64(cnt - group * kSkRows < kSkRows ? cnt - group * kSkRows : kSkRows);

        // Lane l streams weight rows col0 + l % 16 (block 0) and col0 + 16 +
        // l % 16 (block 1) and x row row0 + l % 16 (clamped to the group's
        // last row: its results are not stored).
        const int r = lane % 16;
        const int q = lane / 16;
        const u32x4* wrow = w + ((int64_t)e * n + col0 + r) * kv;
        const int64_t block_stride = 16 * kv;
        const u32x4* xrow = x + (row0 + (r < rows ? r : rows - 1)) * kv;

        f32x4 acc[2] = {f32x4{}, f32x4{}};
        Chunk ring[kSkDepth];
        // Chunks past the last are loaded as the last one and not summed.
        static_for<0, kSkDepth>([&](auto d) {
            constexpr int D = decltype(d)::value;
            load_chunk(ring[D], wrow, block_stride, xrow, D < nchunks ? D : nchunks - 1, q);
        });
        // Whole rounds while the next round is whole too: no branch between
        // the loads and their use, so each wait is for exactly one chunk.
        int64_t c0 = 0;
        for (; c0 + 2 * kSkDepth <= nchunks; c0 += kSkDepth) {
            static_for<0, kSkDepth>([&](auto d) {
                constexpr int D = decltype(d)::value;
                mma_chunk(acc, ring[D]);
                load_chunk(ring[D], wrow, block_stride, xrow, c0 + kSkDepth + D, q);
            });
        }
        for (; c0 < nchunks; c0 += kSkDepth) {
            static_for<0, kSkDepth>([&](auto d) {
                constexpr int D = decltype(d)::value;
                const int64_t c = c0 + D;
                if (c < nchunks) mma_chunk(acc, ring[D]);
                const int64_t nc = c + kSkDepth < nchunks ? c + kSkDepth : nchunks - 1;
                if (c0 + kSkDepth < nchunks) load_chunk(ring[D], wrow, block_stride, xrow, nc, q);
            });
        }

        // Epilogue: lane l holds x row l % 16, columns 4q .. 4q + 3 of each block.
        if (r < rows) {
            uint16_t* yrow = y + (row0 + r) * n + col0 + 4 * q;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t lo2 = bf16_rne(acc[b][0]) | (bf16_rne(acc[b][1]) << 16);
                const uint32_t hi2 = bf16_rne(acc[b][2]) | (bf16_rne(acc[b][3]) << 16);
                *reinterpret_cast<uint2*>(yrow + 16 * b) = make_uint2(lo2, hi2);
            }
        }
    }
}

}  // namespace

hipError_t launch_grouped_gemm_skinny(const GemmArgs& a, int num_cus, hipStream_t stream) {
    // Persistent grid of the workgroups that fit at once; each wave walks its items.
    const int64_t blocks = (int64_t)num_cus * 3;  // three workgroups per CU fit (142 VGPRs)
    hipLaunchKernelGGL(grouped_gemm_skinny_kernel, dim3((unsigned)blocks), dim3(kSkThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(a.x), reinterpret_cast<const u32x4*>(a.w), a.offsets,
                       reinterpret_cast<uint16_t*>(a.y), a.num_experts, a.max_rows, a.n, a.k);
    return hipGetLastError();
}

}  // namespace moe
