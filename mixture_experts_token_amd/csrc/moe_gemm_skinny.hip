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
// and up to 16 of its x rows and streams those weight rows through a private
// pair of LDS stages (no workgroup barrier): a stage is 512 contiguous bytes
// (256 k) of each of the 32 rows, loaded straight into LDS two rows per
// instruction, and the MFMA fragments are read back from it.  Weight rows
// read 64 bytes at a time straight into the MFMA operand layout (16 rows per
// instruction) streamed at 5.1 TB/s at N=1; the same bytes read as long
// contiguous runs reach 6.7 TB/s.  The x fragments of a stage are loaded into
// registers with its weights.  Experts with more than 16 rows take several
// row groups, each streaming the weight rows again.
//
// With at most one or two rows per expert on average a second kernel takes over
// (grouped_gemm_rowstream_kernel, below): one wave reads 8 whole weight rows
// front to back and multiplies them with up to two or four x rows by bf16 dot
// products, without LDS or matrix cores, so every HBM stream is sequential.
//
// MFMA operands (v_mfma_f32_16x16x32_bf16, weight fragment first): for the
// k half h (32 k) of a 64-wide chunk, lane l holds 8 consecutive k (k-vector
// 4h + l / 16 of the chunk) of weight row l % 16 of a 16-row block and of x
// row l % 16; lane l's 4 results are x row l % 16, output columns
// 4 (l / 16) .. 4 (l / 16) + 3 of the block.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "moe_launch.h"
#include "moe_gemm_device.h"
#include "moe_plan.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One configuration of the streaming kernel: COLS weight rows per wave
// (COLS / 16 MFMA blocks), SEG 16-byte k-vectors of each row per stage (SEG
// * 16 contiguous bytes), STAGES LDS stages per wave, WAVES waves per
// workgroup (one workgroup per CU: the stages of its waves fill the LDS).
template <int COLS, int SEG, int STAGES, int WAVES>
struct SkShape {
    static constexpr int kCols = COLS;
    static constexpr int kBlocks = COLS / 16;
    static constexpr int kSeg = SEG;
    static constexpr int kStages = STAGES;
    static constexpr int kWaves = WAVES;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kChunks = SEG / 8;                 // 64-wide k chunks per stage
    static constexpr int kStageVecs = COLS * SEG;           // 16-byte vectors per stage
    static constexpr int kRowsPerLoad = 64 / SEG;           // stage rows one direct-to-LDS load covers
    static constexpr int kLoadsW = kStageVecs / 64;         // direct-to-LDS loads per stage (1 KiB each)
    static constexpr int kLoadsX = 2 * kChunks;             // x fragment loads per stage
    static constexpr int kLoads = kLoadsW + kLoadsX;        // vector-memory operations per stage
    static_assert(COLS % 16 == 0 && SEG >= 16 && SEG <= 64 && 64 % SEG == 0, "stage layout");
    static_assert((STAGES - 1) * kLoads < 64, "the stages in flight fit the vector-memory counter");
    static_assert(WAVES * STAGES * kStageVecs * 16 <= 136 * 1024, "the stages of a workgroup fit the LDS");
};

constexpr int kSkRows = 16;  // x rows per wave (one row group)

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

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they retire in issue order).
template <int N>
__device__ __forceinline__ void sk_wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS slot of k-vector v of stage row `row`: the low four bits are
// XOR-swizzled by the row, so the 16 rows that a 16-lane phase of a fragment
// read touches (same v, a row pitch of a multiple of 256 bytes) fall on 16
// different 16-byte bank groups.  Its own inverse in v.
__device__ __forceinline__ int sk_slot(int row, int v) { return v ^ (row & 15); }

template <typename S>
struct XStage {
    u32x4 f[S::kChunks][2];  // chunk c, k half h
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Stage `st` of this wave's item into `buf` (its LDS stage) and `xs`: load i
// covers stage rows kRowsPerLoad * i ..., lane L writing slot L % SEG of row
// kRowsPerLoad * i + L / SEG, i.e. reading k-vector sk_slot(row, L % SEG) of
// the row's segment.  k-vectors past the row's end (a partial last stage)
// re-read its last vector; the chunks they fall in are not summed.
template <typename S>
__device__ __forceinline__ void sk_issue_stage(u32x4* buf, XStage<S>& xs, const u32x4* __restrict__ wbase,
                                               const u32x4* __restrict__ xrow, int64_t kv, int64_t st, int lane) {
    const int q = lane / 16;
#pragma unroll
    for (int i = 0; i < S::kLoadsW; ++i) {
        const int row = S::kRowsPerLoad * i + lane / S::kSeg;
        const int64_t v = st * S::kSeg + sk_slot(row, lane % S::kSeg);
        __builtin_amdgcn_global_load_lds(wbase + row * kv + (v < kv ? v : kv - 1), buf + i * 64, 16, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < S::kChunks; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t v = st * S::kSeg + c * 8 + 4 * h + q;
            xs.f[c][h] = xrow[v < kv ? v : kv - 1];
        }
}

// The weight fragments of one chunk (2 blocks x 2 k halves) as explicit
// ds_read_b128 and the wait for them, in one asm statement: the compiler does
// not see them as LDS reads, so it adds no wait for the direct-to-LDS loads of
// the other stages still in flight (the caller waits for this stage's loads
// explicitly).  Early-clobber outputs: no destination shares a register with
// an address still to be read.
__device__ __forceinline__ void sk_read4(uint32_t a00, uint32_t a01, uint32_t a10, uint32_t a11, u32x4& f00,
                                         u32x4& f01, u32x4& f10, u32x4& f11) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f00), "=&v"(f01), "=&v"(f10), "=&v"(f11)
        : "v"(a00), "v"(a01), "v"(a10), "v"(a11)
        : "memory");
}

// The MFMAs of stage `st` (its loads complete): chunk c of the stage is
// summed when it lies before the row's end.
template <typename S>
__device__ __forceinline__ void sk_consume_stage(f32x4 (&acc)[S::kBlocks], const u32x4* buf, const XStage<S>& xs,
                                                 int64_t st, int64_t nchunks, int lane) {
    static_assert(S::kBlocks == 2, "two MFMA blocks per wave");
    const int r = lane % 16;
    const int q = lane / 16;
    const uint32_t base = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int c = 0; c < S::kChunks; ++c) {
        if (st * S::kChunks + c >= nchunks) break;  // the same for the whole wave
        uint32_t a[S::kBlocks][2];
#pragma unroll
        for (int b = 0; b < S::kBlocks; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                a[b][h] = base + (uint32_t)(((b * 16 + r) * S::kSeg + sk_slot(r, c * 8 + 4 * h + q)) * 16);
        u32x4 f[S::kBlocks][2];
        sk_read4(a[0][0], a[0][1], a[1][0], a[1][1], f[0][0], f[0][1], f[1][0], f[1][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < S::kBlocks; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f[b][h]),
                                                                 __builtin_bit_cast(bf16x8, xs.f[c][h]), acc[b], 0,
                                                                 0, 0);
    }
}

// Work item = (expert, row group of 16 rows, block of COLS output columns);
// items of one expert are row-group major, so the column blocks of a row
// group run on neighbouring waves (one CU) and share its x rows in cache.
template <typename S>
__global__ __launch_bounds__(S::kThreads) void grouped_gemm_skinny_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n, int64_t k) {
    constexpr int kThreads = S::kThreads;
    // The LDS stages of every wave, written only by direct-to-LDS loads and
    // read only by asm fragment reads.
    __shared__ __attribute__((aligned(1024))) u32x4 stage_s[S::kWaves][S::kStages][S::kStageVecs];
    __shared__ int64_t item_pre[kMaxExperts + 1];
    __shared__ int64_t part[kThreads / 64];  // per-wave totals of the item prefix
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int64_t nblocks = n / S::kCols;
    const int64_t kv = k / 8;  // 16-byte vectors per row
    const int64_t nchunks = k / 64;

    // Items per expert and their prefix; the offsets are checked as in the
    // tiled kernel (the permute writes -1 everywhere when it rejected an id).
    constexpr int kPer = (kMaxExperts + kThreads - 1) / kThreads;
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
    int64_t total;
    int64_t excl = block_exclusive_prefix64<kThreads>(sum, part, total);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < num_experts) item_pre[e] = excl;
        excl += cnt_t[q];
    }
    if (tid == 0) item_pre[num_experts] = total;
    if (__syncthreads_or(bad)) return;  // also publishes item_pre
    const int64_t total_waves = (int64_t)gridDim.x * S::kWaves;

    for (int64_t id = (int64_t)blockIdx.x * S::kWaves + wave; id < total; id += total_waves) {
        int lo = 0, hi = num_experts - 1;  // last expert with item_pre[e] <= id
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (item_pre[mid] <= id) lo = mid;
            else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int64_t local = id - item_pre[e];
        const int64_t group = local / nblocks;
        const int64_t col0 = uniform64((local - group * nblocks) * S::kCols);
        const int64_t row0 = uniform64(off[e] + group * kSkRows);
        const int64_t cnt = off[e + 1] - off[e];
        const int rows = (int)uniform64(cnt - group * kSkRows < kSkRows ? cnt - group * kSkRows : kSkRows);

        // The wave streams weight rows col0 .. col0 + COLS - 1 of expert e;
        // lane l's x fragments come from x row row0 + l % 16 (clamped to the
        // group's last row: its results are not stored).
        const int r = lane % 16;
        const int q = lane / 16;
        const u32x4* wbase = w + ((int64_t)e * n + col0) * kv;
        const u32x4* xrow = x + (row0 + (r < rows ? r : rows - 1)) * kv;
        const int64_t nst = (nchunks + S::kChunks - 1) / S::kChunks;

        // STAGES stages in flight while the oldest is summed.  Every step
        // issues a whole stage (past the last one, the last again, never
        // summed), so each wait is for exactly one stage's loads.
        f32x4 acc[S::kBlocks];
#pragma unroll
        for (int b = 0; b < S::kBlocks; ++b) acc[b] = f32x4{};
        XStage<S> xs[S::kStages];
        static_for<0, S::kStages>([&](auto d) {
            constexpr int D = decltype(d)::value;
            sk_issue_stage<S>(stage_s[wave][D], xs[D], wbase, xrow, kv, D < nst ? D : nst - 1, lane);
        });
        for (int64_t st = 0; st < nst; st += S::kStages) {
            static_for<0, S::kStages>([&](auto d) {
                constexpr int D = decltype(d)::value;
                sk_wait_vmem<(S::kStages - 1) * S::kLoads>();
                if (D == 0 || st + D < nst) sk_consume_stage<S>(acc, stage_s[wave][D], xs[D], st + D, nchunks, lane);
                const int64_t nx = st + D + S::kStages;
                sk_issue_stage<S>(stage_s[wave][D], xs[D], wbase, xrow, kv, nx < nst ? nx : nst - 1, lane);
            });
        }
        // The last stages' re-reads land before the next item's loads reuse
        // the stages.
        sk_wait_vmem<0>();

        // Epilogue: lane l holds x row l % 16, columns 4q .. 4q + 3 of each block.
        if (r < rows) {
            uint16_t* yrow = y + (row0 + r) * n + col0 + 4 * q;
#pragma unroll
            for (int b = 0; b < S::kBlocks; ++b) {
                const uint32_t lo2 = bf16_rne(acc[b][0]) | (bf16_rne(acc[b][1]) << 16);
                const uint32_t hi2 = bf16_rne(acc[b][2]) | (bf16_rne(acc[b][3]) << 16);
                *reinterpret_cast<uint2*>(yrow + 16 * b) = make_uint2(lo2, hi2);
            }
        }
    }
}

template <typename S>
hipError_t launch_skinny(const GemmArgs& a, int num_cus, hipStream_t stream) {
    hipLaunchKernelGGL(grouped_gemm_skinny_kernel<S>, dim3((unsigned)num_cus), dim3(S::kThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(a.x), reinterpret_cast<const u32x4*>(a.w), a.offsets,
                       reinterpret_cast<uint16_t*>(a.y), a.num_experts, a.max_rows, a.n, a.k);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Row-streaming kernel for experts with one to four rows (decode at a token
// or a few): one wave owns COLS (8) consecutive weight rows of one expert (a
// single contiguous COLS x k block of w) and up to XR (2 or 4) of its x rows, and reads
// the block front to back, 1 KiB per load, RA weight rows in flight.  Each lane
// multiplies its 16-byte weight vectors with the matching x vectors (held in
// registers for the whole item) by bf16 dot products into fp32, and a row's 64
// lane sums are added across the wave (DPP) when the row ends.  No LDS and no
// matrix cores: with one x row the matrix cores would idle on a 16-row tile,
// and streaming each weight row whole keeps the HBM reads sequential, which
// the 16-row fragment layout of the other kernels cannot.
// KV64 = k / 512: loads per weight row (k a multiple of 512, at most 8192).
// ----------------------------------------------------------------------------
constexpr int kRsCols = 8;      // weight rows (output columns) per item
constexpr int kRsThreads = 256;
constexpr int kRsMaxKv64 = 16;  // k <= 8192
constexpr int kRsMaxKv64X4 = 8; // k <= 4096 with four x rows per item

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The lanes' elements are copied out before the bit cast: a bit cast of the
// vector element itself (wv[p]) compiled to element 0 for every p.
__device__ __forceinline__ float dot8(const u32x4& wv, const u32x4& xv, float acc) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t wp = wv[p], xp = xv[p];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp), __builtin_bit_cast(bf16x2, xp), acc,
                                              false);
    }
    return acc;
}

// Sum over the 64 lanes of a wave (every lane active): the DPP inclusive scan
// of the permute's index passes on float bits (row shifts 1, 2, 4, 8, then the
// broadcasts of lanes 15 and 31; lanes without a source add +0), lane 63's
// value read out.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int KV64, int RA, int COLS, int XR>
__global__ __launch_bounds__(kRsThreads) void grouped_gemm_rowstream_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n) {
    static_assert(COLS <= 64 && COLS % RA == 0, "one result lane per weight row; whole rounds of RA rows");
    constexpr int kWaves = kRsThreads / 64;
    constexpr int kv = KV64 * 64;  // 16-byte vectors per row
    __shared__ int64_t item_pre[kMaxExperts + 1];
    __shared__ int64_t part[kRsThreads / 64];  // per-wave totals of the item prefix
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int64_t nblocks = n / COLS;

    // Items per expert and their prefix, as in the other grouped GEMM kernels.
    constexpr int kPer = (kMaxExperts + kRsThreads - 1) / kRsThreads;
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
            cnt_t[q] = cnt > 0 ? (cnt + XR - 1) / XR * nblocks : 0;
        }
        sum += cnt_t[q];
    }
    if (tid == 0) bad |= off[0] != 0 || off[num_experts] > max_rows;
    int64_t total;
    int64_t excl = block_exclusive_prefix64<kRsThreads>(sum, part, total);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < num_experts) item_pre[e] = excl;
        excl += cnt_t[q];
    }
    if (tid == 0) item_pre[num_experts] = total;
    if (__syncthreads_or(bad)) return;  // also publishes item_pre
    const int64_t total_waves = (int64_t)gridDim.x * kWaves;

    for (int64_t id = (int64_t)blockIdx.x * kWaves + wave; id < total; id += total_waves) {
        int lo = 0, hi = num_experts - 1;  // last expert with item_pre[e] <= id
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (item_pre[mid] <= id) lo = mid;
            else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int64_t local = id - item_pre[e];
        const int64_t group = local / nblocks;
        const int64_t col0 = uniform64((local - group * nblocks) * COLS);
        const int64_t row0 = uniform64(off[e] + group * XR);
        const int64_t cnt = off[e + 1] - off[e];
        const int rows = (int)uniform64(cnt - group * XR < XR ? cnt - group * XR : XR);

        // x vectors i * 64 + lane of the item's rows (a missing second row
        // repeats the first: its sums are not stored).
        u32x4 xr[XR][KV64];
#pragma unroll
        for (int r = 0; r < XR; ++r)
#pragma unroll
            for (int i = 0; i < KV64; ++i) xr[r][i] = x[(row0 + (r < rows ? r : 0)) * kv + i * 64 + lane];
        // Weight rows col0 .. col0 + COLS - 1: one contiguous block.
        const u32x4* wb = w + ((int64_t)e * n + col0) * kv + lane;
        u32x4 ring[RA][KV64];
#pragma unroll
        for (int a = 0; a < RA; ++a)
#pragma unroll
            for (int i = 0; i < KV64; ++i) {
                ring[a][i] = __builtin_nontemporal_load(wb + (a * KV64 + i) * 64);
                __builtin_amdgcn_sched_barrier(0);  // issued in the loop's order (see below)
            }

        float res[XR] = {};
        for (int j0 = 0; j0 < COLS; j0 += RA) {
#pragma unroll
            for (int a = 0; a < RA; ++a) {
                const int j = j0 + a;
                // Row j + RA goes into the slots row j frees; past the block
                // the last row is read again (not summed), so every step
                // issues the same loads and each wait is for one row.
                const int jn = j + RA < COLS ? j + RA : COLS - 1;
                float acc[XR] = {};
#pragma unroll
                for (int i = 0; i < KV64; ++i) {
                    // Use a vector, then refill its registers: a sliding
                    // window of RA * KV64 loads.  The scheduling barrier keeps
                    // the compiler from hoisting the refills above the uses,
                    // which would make it wait for the whole window first.
#pragma unroll
                    for (int r = 0; r < XR; ++r) acc[r] = dot8(ring[a][i], xr[r][i], acc[r]);
                    ring[a][i] = __builtin_nontemporal_load(wb + ((int64_t)jn * KV64 + i) * 64);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int r = 0; r < XR; ++r) {
                    const float t = wave_sum(acc[r]);
                    if (lane == j) res[r] = t;
                }
            }
        }
        // Lane c holds output column col0 + c of each x row.
        if (lane < COLS) {
#pragma unroll
            for (int r = 0; r < XR; ++r)
                if (r < rows) y[(row0 + r) * n + col0 + lane] = (uint16_t)bf16_rne(res[r]);
        }
    }
}

// RA = rows in flight: about 16 loads (16 KiB) per wave, a power of two that
// divides the 8 rows of an item.  Measured at the DSv3 decode shape (N=1, k
// 7168, 14 loads per row, 32 rows per item): one row in flight 70.5 us, two
// 73.2.  Rows per item, 32 / 16 / 8 / 4 (same box): DSv3 N=1 70.5 / 70.4 /
// 69.8 / 69.6 us, N=16 860 / 861 / 859 / 857; Mixtral N=1 72.1 / 80.0 / 70.8 /
// 69.9, N=4 182 / 187 / 171 / 169; Qwen3 N=1 13.9 / 10.5 / 10.1 / 9.8, N=16
// 94.5 / 90.5 / 82.6 / 84.3: more, shorter items fill the CUs when the experts
// with rows have few weight rows between them, and 8 rows re-read each x row
// from L2 half as often as 4.
template <int KV64, int XR>
hipError_t launch_rowstream_kx(const GemmArgs& a, int num_cus, hipStream_t stream) {
    constexpr int RA0 = KV64 > 8 ? 1 : KV64 > 4 ? 2 : KV64 > 2 ? 4 : KV64 > 1 ? 8 : 16;
    constexpr int RA = RA0 < kRsCols ? RA0 : kRsCols;
    const int64_t blocks = (int64_t)num_cus * 2;  // two workgroups per CU fit (at most 215 VGPRs)
    hipLaunchKernelGGL((grouped_gemm_rowstream_kernel<KV64, RA, kRsCols, XR>), dim3((unsigned)blocks),
                       dim3(kRsThreads), 0, stream, reinterpret_cast<const u32x4*>(a.x),
                       reinterpret_cast<const u32x4*>(a.w), a.offsets, reinterpret_cast<uint16_t*>(a.y),
                       a.num_experts, a.max_rows, a.n);
    return hipGetLastError();
}

// Four x rows per item only up to k 4096 (KV64 8): more x registers would
// not leave two waves per SIMD.
template <int KV64>
hipError_t launch_rowstream_kc(const GemmArgs& a, int num_cus, int x_rows, hipStream_t stream) {
    if constexpr (KV64 <= kRsMaxKv64X4) {
        if (x_rows == 4) return launch_rowstream_kx<KV64, 4>(a, num_cus, stream);
    }
    return launch_rowstream_kx<KV64, 2>(a, num_cus, stream);
}

}  // namespace

bool gemm_rowstream_fits(int64_t k, int x_rows) {
    return k % 512 == 0 && k <= 512 * (x_rows == 4 ? kRsMaxKv64X4 : kRsMaxKv64);
}

// Persistent grid, one workgroup per CU (its waves' LDS stages fill the LDS);
// each wave walks its items.  Stages of 512 bytes of 32 weight rows, two per
// wave, four waves: DSv3 decode N=1 83.9 us; 1 KiB of 16 rows 86.2 us, 512
// bytes of 16 rows in four stages 84.9, 256 bytes of 32 rows in four stages
// 85.1; two waves per CU with 1 KiB of 32 rows 89.4, three 512-byte stages
// 88.8 (the previous kernel, 64 bytes of 16 rows per load straight into MFMA
// operands: 90.7).
hipError_t launch_grouped_gemm_skinny(const GemmArgs& a, int num_cus, hipStream_t stream) {
    return launch_skinny<SkShape<32, 32, 2, 4>>(a, num_cus, stream);
}

hipError_t launch_grouped_gemm_rowstream(const GemmArgs& a, int num_cus, int x_rows, hipStream_t stream) {
    switch (a.k / 512) {
        case 1: return launch_rowstream_kc<1>(a, num_cus, x_rows, stream);
        case 2: return launch_rowstream_kc<2>(a, num_cus, x_rows, stream);
        case 3: return launch_rowstream_kc<3>(a, num_cus, x_rows, stream);
        case 4: return launch_rowstream_kc<4>(a, num_cus, x_rows, stream);
        case 5: return launch_rowstream_kc<5>(a, num_cus, x_rows, stream);
        case 6: return launch_rowstream_kc<6>(a, num_cus, x_rows, stream);
        case 7: return launch_rowstream_kc<7>(a, num_cus, x_rows, stream);
        case 8: return launch_rowstream_kc<8>(a, num_cus, x_rows, stream);
        case 9: return launch_rowstream_kc<9>(a, num_cus, x_rows, stream);
        case 10: return launch_rowstream_kc<10>(a, num_cus, x_rows, stream);
        case 11: return launch_rowstream_kc<11>(a, num_cus, x_rows, stream);
        case 12: return launch_rowstream_kc<12>(a, num_cus, x_rows, stream);
        case 13: return launch_rowstream_kc<13>(a, num_cus, x_rows, stream);
        case 14: return launch_rowstream_kc<14>(a, num_cus, x_rows, stream);
        case 15: return launch_rowstream_kc<15>(a, num_cus, x_rows, stream);
        case 16: return launch_rowstream_kc<16>(a, num_cus, x_rows, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
