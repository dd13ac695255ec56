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
//   * output tiles of 128 rows x 256 columns, a workgroup of 8 waves, each
//     wave a 64 x 64 block of 2 x 2 v_mfma_f32_32x32x16_bf16 tiles, three LDS
//     stages (one workgroup per CU); 128 x 128 tiles of 4 waves, two stages,
//     two workgroups per CU when n is not a multiple of 256; k advances 64
//     per step;
//   * both operands go from global memory straight into LDS (16 bytes per
//     lane, no register round trip), 128-byte rows with the 16-byte k-vectors
//     of row r stored in slot kvec ^ (r % 8) ^ (bit 3 of r), so the fragment
//     reads of 16 consecutive rows hit every bank once; the wide tiles load through buffer
//     resources (one lane offset register per operand, row group and k step
//     in the scalar offset) and spread a step's loads over its four 16-wide k
//     slices instead of issuing them all after the barrier;
//   * the pipeline's waits are explicit: before step ks each wave waits only
//     for its own loads of step ks (those of ks + 1 stay in flight), then one
//     barrier; fragment reads are explicit ds_read_b128 so the compiler adds
//     no wait for loads still landing in other stages;
//   * the tile list lives on the device: the offsets come from the permute, so
//     every workgroup derives the per-expert tile counts from them (prefix in
//     LDS) and walks tiles persistently.  Order: per expert, groups of 8 row
//     tiles (a remainder of 1-3 tiles joins the last group), all column tiles
//     of a group, row tiles fastest -- a group's rows
//     and a column tile's weights are reused while they are cached; the
//     concurrently running tiles are split into one contiguous chunk per XCD
//     (workgroups are dispatched round-robin over the 8 XCDs), so each XCD's
//     L2 sees neighbouring tiles.

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
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kGroupM = 8;             // row tiles per group in the tile order (the last group: 1-11)
constexpr int kXcds = 8;

// Tile shape: BM x BN outputs per workgroup of WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 32 x 32 MFMA tiles; STAGES LDS buffers per
// operand; PER_CU workgroups resident per compute unit (registers and LDS are
// budgeted for that many).  FAST: loads through buffer resources spread over
// the k slices, fragment reads as explicit ds_read_b128 (lds_read_slice); otherwise
// global_load_lds issued together after the barrier and fragment reads left
// to the compiler.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int PER_CU_, bool FAST_>
struct GemmShape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, PER_CU = PER_CU_;
    static constexpr bool FAST = FAST_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int MT = kWaveM / 32, NT = kWaveN / 32;
    // direct-to-LDS instructions per wave per k-step (8 rows of 128 bytes each)
    static constexpr int kLoadsPerStep = (BM + BN) / kWaves / 8;
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile is whole 32 x 32 MFMA tiles");
    static_assert(BM % (kWaves * 8) == 0 && BN % (kWaves * 8) == 0, "every wave loads whole 8-row groups");
    static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
    // compiler-scheduled fragment reads would wait for every load in flight
    static_assert(FAST || STAGES == 2, "a third stage needs the explicit fragment reads");
    static_assert(kLoadsPerStep <= 31, "vector-memory count of one step fits the wait immediate");
    static constexpr int kLdsBytes = STAGES * (BM + BN) * kBK * 2;
    static_assert(kLdsBytes * PER_CU <= 150 * 1024, "stages of every resident workgroup fit the 160 KiB LDS");
};

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Wait until at most `n` of this wave's vector-memory operations are
// outstanding (they retire in issue order), leaving the LDS and export
// counters alone.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the k-step pipeline: this wave's LDS reads are
// complete (lgkmcnt) before it arrives, and no memory access is moved across
// it.  Written as one asm statement because the compiler's own release fence
// would also wait for every direct-to-LDS load in flight (vmcnt(0)), which is
// exactly the overlap the pipeline exists for; the direct-to-LDS loads a step
// needs are waited for explicitly (wait_vmem) before the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A value every lane of the wave holds, moved into a scalar register (the
// compiler cannot prove uniformity of values read from LDS).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
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
    // Groups of kGroupM row tiles; a remainder of 1-3 row tiles joins the last
    // group, so that no short group streams all of the expert's weight column
    // tiles again for one to three row tiles (a longer remainder keeps its own
    // group: larger groups fetch more row bytes per column tile).
    const int64_t ng = mt % kGroupM <= 3 && mt / kGroupM > 0 ? mt / kGroupM : (mt + kGroupM - 1) / kGroupM;
    const int64_t g0 = local / (kGroupM * n_tiles);
    const int64_t g = g0 < ng - 1 ? g0 : ng - 1;
    const int64_t gsize = g == ng - 1 ? mt - g * kGroupM : kGroupM;
    const int64_t r = local - g * kGroupM * n_tiles;
    const int64_t nt = r / gsize;
    const int64_t mi = g * kGroupM + (r - nt * gsize);
    TileCoord c;
    c.expert = __builtin_amdgcn_readfirstlane(e);
    c.row0 = uniform64(off[e] + mi * BM);
    c.rows = uniform64(cnt - mi * BM < BM ? cnt - mi * BM : BM);
    c.col0 = uniform64(nt * BN);
    return c;
}

// LDS slot of k-vector kvec of tile row `row`: the 16-byte k-vectors of a
// 128-byte row are XOR-swizzled by the row.  A 128-byte row spans half of the
// LDS banks, so two rows share a bank line and a 16-lane phase of a 16-byte
// read touches 16 consecutive rows: the row's bit 3 flips the slot as well, so
// rows r and r + 8 (same row % 8, same bank half) land in different banks.
// With only row % 8, half of the LDS cycles of the fragment reads were bank
// conflicts (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = 0.50 at the Mixtral
// shape); with this slot none (0.00), grouped GEMM 2048 -> 1989 us.
__device__ __forceinline__ int kslot(int row, int kvec) { return kvec ^ (row % 8) ^ ((row / 8) & 1); }

// Operand tiles (ROWS rows x 64 bf16 = 128 bytes per row per k-step) go from
// global memory straight into LDS, one 1 KiB instruction (8 rows) at a time:
// lane L of an instruction writes slot L % 8 of row L / 8 of its group and
// reads the k-vector of that row that belongs in that slot (kslot is its own
// inverse in kvec).
// One 8-row group: `row` is this lane's row (group start + L / 8), `srow` the
// row it reads (clamped into the valid rows), `lds_group` the group's LDS rows.
__device__ __forceinline__ void group_to_lds(__bf16* lds_group, const u32x4* __restrict__ src_row0,
                                             int64_t row_stride_vecs, int row, int srow, int64_t kvec0, int lane) {
    const u32x4* g = src_row0 + (int64_t)srow * row_stride_vecs + kvec0 + kslot(row, lane % 8);
    __builtin_amdgcn_global_load_lds(g, lds_group, 16, 0, 0);
}

// One 8-row group of the same load through a buffer resource whose base is
// the tile's first row: lane L reads row L / 8 of the group, k-vector
// kslot(group row + L / 8, L % 8) (groups are 8-aligned); the group row
// and the k step go into the scalar offset.  With kClamp, rows past
// rows_valid re-read the last valid row (the group start is clamped too, so
// the lane offset never goes negative): every step issues the same number of
// loads, which the vector-memory waits count on.
template <bool kClamp>
__device__ __forceinline__ void group_to_lds_buf(__bf16* lds_group, __amdgpu_buffer_rsrc_t rsrc, int stride_bytes,
                                                 int grow, int rows_valid, int step, int lane) {
    const int chunk = kslot(grow + lane / 8, lane % 8) * 16;
    int g0 = grow, r = lane / 8;
    if (kClamp) {
        g0 = grow < rows_valid ? grow : rows_valid - 1;
        r = (grow + r < rows_valid ? grow + r : rows_valid - 1) - g0;
    }
    const int soffset = __builtin_amdgcn_readfirstlane(g0 * stride_bytes + step * (kBK * 2));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_group, 16,
                                             r * stride_bytes + chunk, soffset, 0, 0);
}

// Fragment of 8 consecutive k (k-vector kvec) of tile row `row`.
__device__ __forceinline__ bf16x8 lds_frag(const __bf16* lds, int row, int kvec) {
    return *reinterpret_cast<const bf16x8*>(lds + row * kBK + kslot(row, kvec) * 8);
}

// LDS byte address of the 16-byte fragment vector (row, kvec) of a stage: a
// generic address of LDS memory holds the LDS byte offset in its low 32 bits.
__device__ __forceinline__ uint32_t lds_frag_addr(const __bf16* lds, int row, int kvec) {
    return (uint32_t)(uintptr_t)(lds + row * kBK + kslot(row, kvec) * 8);
}

// The four fragment reads of one 16-wide k slice (two row fragments, two
// weight fragments) as explicit ds_read_b128, and the wait for them, in one
// asm statement.  The compiler does not see these as LDS reads, so it adds no
// wait for direct-to-LDS loads still in flight into other stages (it cannot
// tell the stages apart and would wait for all of them); the caller orders
// the statement after the barrier that publishes its stage.  The wait sits in
// the same statement so that the destination registers are written before
// the compiler regards them as defined, and the outputs are early-clobber so
// that no destination shares a register with an address still to be read.
__device__ __forceinline__ void lds_read_slice(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, u32x4& fa0,
                                               u32x4& fa1, u32x4& fb0, u32x4& fb1) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa0), "=&v"(fa1), "=&v"(fb0), "=&v"(fb1)
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
        : "memory");
}

// A copy the compiler cannot see through or move out of a loop: per-lane
// values derived from it are recomputed where they are used instead of being
// hoisted out of the k-loop and kept live across it.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// The same for a wave whose second row fragment holds no rows of the tile:
// one row fragment and the two weight fragments.
__device__ __forceinline__ void lds_read_slice3(uint32_t a0, uint32_t b0, uint32_t b1, u32x4& fa0, u32x4& fb0,
                                                u32x4& fb1) {
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %4\n\t"
        "ds_read_b128 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa0), "=&v"(fb0), "=&v"(fb1)
        : "v"(a0), "v"(b0), "v"(b1)
        : "memory");
}

template <int I>
using Int = std::integral_constant<int, I>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(Int<I>{});
        static_for<I + 1, N>(f);
    }
}

// Persistent grouped GEMM.  The MFMA takes the weight fragment as its first
// operand and the row fragment as its second, so a lane's 16 results are 4
// runs of 4 consecutive output columns of one row (8-byte stores in the
// epilogue).
template <typename S>
__global__ __launch_bounds__(S::kThreads, S::PER_CU) void grouped_gemm_bf16_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ w, const int64_t* __restrict__ off,
    uint16_t* __restrict__ y, int num_experts, int64_t max_rows, int64_t n, int64_t k) {
    constexpr int BM = S::BM, BN = S::BN, MT = S::MT, NT = S::NT, STAGES = S::STAGES;
    constexpr int kThreads = S::kThreads;
    // The tile's results go out through the idle weight stages when a stage
    // holds 64 rows of the tile (128 x 256 tiles, two waves down the rows).
    constexpr bool kStagedOut = S::FAST && BM == 128 && BN == 256 && S::WM == 2 && BN * kBK * 2 == 64 * 512 &&
                                (BM / S::kWaves) % 2 == 0 && 64 % (BM / S::kWaves) == 0;
    // Each stage of each operand is its own LDS object, so the compiler's
    // wait tracking can tell a stage being filled from the ones being read.
    constexpr int kA2 = STAGES > 2 ? BM * kBK : 8, kB2 = STAGES > 2 ? BN * kBK : 8;
    __shared__ __attribute__((aligned(1024))) __bf16 a_s0[BM * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 a_s1[BM * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 a_s2[kA2];
    __shared__ __attribute__((aligned(1024))) __bf16 b_s0[BN * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 b_s1[BN * kBK];
    __shared__ __attribute__((aligned(1024))) __bf16 b_s2[kB2];
    __shared__ int64_t tile_pre[kMaxExperts + 1];
    __shared__ int64_t part[kThreads / 64];  // per-wave totals of the item prefix

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = wave / S::WN, wn = wave % S::WN;  // this wave's block of the tile
    const int64_t n_tiles = n / BN;
    const int64_t kv = k / 8;                        // 16-byte vectors per row of x / w
    const int stride_bytes = (int)(k * 2);           // k <= 2^20 (checked on the host)

    // The stages are written only by direct-to-LDS loads, which the compiler
    // does not see as stores: one visible store keeps their reads from being
    // folded away as reads of never-written memory.
    if (tid == 0) {
        a_s0[0] = a_s1[0] = a_s2[0] = b_s0[0] = b_s1[0] = b_s2[0] = (__bf16)0.0f;
    }

    // Tile counts per expert and their prefix (each thread takes kPer
    // consecutive experts; a scan over the threads in LDS), and a check of the
    // offsets (the permute writes -1 everywhere when it rejected an id).
    constexpr int kPer = (kMaxExperts + kThreads - 1) / kThreads;
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
    int64_t total;
    int64_t excl = block_exclusive_prefix64<kThreads>(s, part, total);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < num_experts) tile_pre[e] = excl;
        excl += cnt_t[q];
    }
    if (tid == 0) tile_pre[num_experts] = total;
    if (__syncthreads_or(bad)) return;  // also publishes tile_pre

    auto stage_a = [&](auto st) __attribute__((always_inline)) -> __bf16* {
        if constexpr (decltype(st)::value == 0) return a_s0;
        else if constexpr (decltype(st)::value == 1) return a_s1;
        else return a_s2;
    };
    auto stage_b = [&](auto st) __attribute__((always_inline)) -> __bf16* {
        if constexpr (decltype(st)::value == 0) return b_s0;
        else if constexpr (decltype(st)::value == 1) return b_s1;
        else return b_s2;
    };

    // This lane's byte offset of its first fragment (k slice 0) within a stage
    // of the row tile and of the weight tile.
    const uint32_t a_lane_off = lds_frag_addr(a_s0, wm * S::kWaveM + lane % 32, lane / 32) - lds_frag_addr(a_s0, 0, 0);
    const uint32_t b_lane_off = lds_frag_addr(b_s0, wn * S::kWaveN + lane % 32, lane / 32) - lds_frag_addr(b_s0, 0, 0);

    // Persistent walk: iteration i covers tiles [i*G, (i+1)*G), G = gridDim.x;
    // XCD x (blocks b with b % 8 == x) takes the contiguous chunk x*G/8 ...
    const int64_t G = gridDim.x;
    const int64_t per_xcd = G / kXcds;
    const int64_t slot = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    // Each tile's coordinates are worked out during the previous tile (after its
    // first loads are issued), so the dependent LDS search and offset loads are
    // off the path between two tiles.
    TileCoord tc_next{};
    if (slot < total) tc_next = tile_coord<BM, BN>(slot, off, tile_pre, num_experts, n_tiles);
    for (int64_t base = 0; base < total; base += G) {
        const int64_t id = base + slot;
        if (id >= total) break;
        const TileCoord tc = tc_next;
        const u32x4* xrow0 = x + tc.row0 * kv;
        const u32x4* wrow0 = w + ((int64_t)tc.expert * n + tc.col0) * kv;
        const int rows_valid = (int)tc.rows;

        f32x16 acc[MT][NT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x16{};

        // Buffer resources over the tile's rows (raw, 32-bit data format).
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)uniform64((int64_t)xrow0), 0, __builtin_amdgcn_readfirstlane(rows_valid * stride_bytes), 0x00020000);
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)uniform64((int64_t)wrow0), 0, __builtin_amdgcn_readfirstlane(BN * stride_bytes), 0x00020000);

        // Load instructions I0 .. I1 - 1 of one k-step for this wave: its 8-row
        // groups of the row tile first, then those of the weight tile.  Every
        // step issues all kGA + kGB of them (clamped rows instead of skipped
        // groups), which the vector-memory waits count on.
        constexpr int kGA = BM / S::kWaves / 8, kGB = BN / S::kWaves / 8;
        auto load_part = [&](int64_t step, auto st, auto i0, auto i1) __attribute__((always_inline)) {
            static_for<decltype(i0)::value, decltype(i1)::value>([&](auto i) __attribute__((always_inline)) {
                constexpr int ii = decltype(i)::value;
                if constexpr (S::FAST) {
                    if constexpr (ii < kGA) {
                        const int grow = wave * (BM / S::kWaves) + ii * 8;
                        group_to_lds_buf<true>(stage_a(st) + grow * kBK, xr, stride_bytes, grow, rows_valid, (int)step, lane);
                    } else {
                        const int grow = wave * (BN / S::kWaves) + (ii - kGA) * 8;
                        group_to_lds_buf<false>(stage_b(st) + grow * kBK, wr, stride_bytes, grow, BN, (int)step, lane);
                    }
                } else {
                    if constexpr (ii < kGA) {
                        const int row = wave * (BM / S::kWaves) + ii * 8 + lane / 8;
                        const int srow = row < rows_valid ? row : rows_valid - 1;  // clamp: a valid row, result unused
                        group_to_lds(stage_a(st) + (row - lane / 8) * kBK, xrow0, kv, row, srow, step * (kBK / 8), lane);
                    } else {
                        const int row = wave * (BN / S::kWaves) + (ii - kGA) * 8 + lane / 8;
                        group_to_lds(stage_b(st) + (row - lane / 8) * kBK, wrow0, kv, row, row, step * (kBK / 8), lane);
                    }
                }
            });
        };
        // One k-step from stage st: four 16-wide k slices; hook(kk) runs
        // before slice kk's MFMAs (it issues part of the next step's loads).
        // mf: the 32-row fragments of this wave's block that hold rows of the
        // tile (the others' results are never stored, so their MFMAs are skipped).
        auto compute_step = [&](auto st, auto mf, auto&& hook) __attribute__((always_inline)) {
            const __bf16* as = stage_a(st);
            const __bf16* bs = stage_b(st);
            // Explicit fragment addresses: rows 32 apart have the same row % 8
            // and bit 3, so both fragments of an operand share one slot (4 KiB
            // apart); slice kk's slot is slice 0's XOR 2 kk (address bits 5-6).
            // Two opaque per-lane offsets per step, instead of the 16 addresses
            // per stage the compiler kept live through the loop (246 -> 201 VGPRs,
            // Mixtral- / Qwen3- / DSv3-shaped 2-5 % faster, bit-identical).
            const uint32_t a_off = opaque_u32(a_lane_off), b_off = opaque_u32(b_lane_off);
            const uint32_t as_addr = lds_frag_addr(as, 0, 0), bs_addr = lds_frag_addr(bs, 0, 0);
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                const int kvec = kk * 2 + lane / 32;
                bf16x8 af[MT], bfr[NT];
                if constexpr (S::FAST) {
                    static_assert(MT == 2 && NT == 2, "lds_read_slice reads 2 + 2 fragments");
                    u32x4 fa[MT], fb[NT];
                    const uint32_t a0 = as_addr + (a_off ^ (uint32_t)(kk * 32));
                    const uint32_t b0 = bs_addr + (b_off ^ (uint32_t)(kk * 32));
                    if constexpr (decltype(mf)::value == 2) {
                        lds_read_slice(a0, a0 + 32 * kBK * 2, b0, b0 + 32 * kBK * 2, fa[0], fa[1], fb[0], fb[1]);
                    } else if constexpr (decltype(mf)::value == 1) {
                        lds_read_slice3(a0, b0, b0 + 32 * kBK * 2, fa[0], fb[0], fb[1]);
                        fa[1] = fa[0];  // not used
                    } else {
                        fa[0] = fa[1] = fb[0] = fb[1] = u32x4{};  // not used: no MFMAs, no reads
                    }
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) af[mi] = __builtin_bit_cast(bf16x8, fa[mi]);
#pragma unroll
                    for (int ni = 0; ni < NT; ++ni) bfr[ni] = __builtin_bit_cast(bf16x8, fb[ni]);
                } else {
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) af[mi] = lds_frag(as, wm * S::kWaveM + mi * 32 + lane % 32, kvec);
#pragma unroll
                    for (int ni = 0; ni < NT; ++ni) bfr[ni] = lds_frag(bs, wn * S::kWaveN + ni * 32 + lane % 32, kvec);
                }
                hook(kk);
#pragma unroll
                for (int mi = 0; mi < decltype(mf)::value; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NT; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
            }
        };

        // Software pipeline over k-steps: step ks computes from stage
        // ks % STAGES while the loads of the next STAGES - 1 steps are in
        // flight.  Before step ks: this wave's loads of step ks have landed
        // (the ones issued after them may not have), then one LDS barrier --
        // after it every wave's step-ks data is in LDS and every wave is done
        // reading the stage that step ks + STAGES - 1 refills.
        const int64_t ksteps = k / kBK;
        lds_barrier();  // the previous tile is done with every stage
        static_for<0, STAGES - 1>([&](auto st) __attribute__((always_inline)) {
            if (decltype(st)::value < ksteps) load_part(decltype(st)::value, st, Int<0>{}, Int<kGA + kGB>{});
        });
        if (id + G < total) {
            tc_next = tile_coord<BM, BN>(id + G, off, tile_pre, num_experts, n_tiles);
            // computed here, not moved down to its use after the k-loop
            asm volatile("" ::"s"(tc_next.expert), "s"(tc_next.row0), "s"(tc_next.rows), "s"(tc_next.col0));
        }
        // full: the caller knows that step ks + STAGES - 1 exists (no branch on it).
        auto step = [&](int64_t ks, auto st, auto full, auto mf) __attribute__((always_inline)) {
            constexpr int kSt = decltype(st)::value;
            constexpr bool kFull = decltype(full)::value;
            if (STAGES == 3 && (kFull || ks + 1 < ksteps)) wait_vmem<(STAGES == 3 ? 1 : 0) * S::kLoadsPerStep>();
            else wait_vmem<0>();
            lds_barrier();
            constexpr auto nst = Int<(kSt + STAGES - 1) % STAGES>{};
            const int64_t nstep = ks + STAGES - 1;
            if (kFull || nstep < ksteps) {
                if constexpr (S::FAST) {
                    // the next step's loads go out a quarter at a time, one
                    // part before each k slice's MFMAs
                    constexpr int n4 = kGA + kGB;
                    compute_step(st, mf, [&](int kk) __attribute__((always_inline)) {
                        if (kk == 0) load_part(nstep, nst, Int<0>{}, Int<n4 / 4>{});
                        else if (kk == 1) load_part(nstep, nst, Int<n4 / 4>{}, Int<n4 / 2>{});
                        else if (kk == 2) load_part(nstep, nst, Int<n4 / 2>{}, Int<3 * n4 / 4>{});
                        else load_part(nstep, nst, Int<3 * n4 / 4>{}, Int<n4>{});
                    });
                } else {
                    load_part(nstep, nst, Int<0>{}, Int<kGA + kGB>{});
                    __builtin_amdgcn_sched_barrier(0);  // the loads go out before this step's LDS reads
                    compute_step(st, mf, [](int) __attribute__((always_inline)) {});
                }
            } else {
                compute_step(st, mf, [](int) __attribute__((always_inline)) {});
            }
        };
        // Whole rounds of STAGES steps (those in which every step refills a
        // stage have no branch inside), then the last ksteps % STAGES steps
        // (stages 0, 1, ... again).
        auto k_loop = [&](auto mf) __attribute__((always_inline)) {
            int64_t ks = 0;
            for (; ks + 2 * STAGES - 1 <= ksteps; ks += STAGES)
                static_for<0, STAGES>([&](auto st) __attribute__((always_inline)) {
                    step(ks + decltype(st)::value, st, Int<1>{}, mf);
                });
            for (; ks + STAGES <= ksteps; ks += STAGES)
                static_for<0, STAGES>([&](auto st) __attribute__((always_inline)) {
                    step(ks + decltype(st)::value, st, Int<0>{}, mf);
                });
            if (ks < ksteps) step(ks, Int<0>{}, Int<0>{}, mf);
            if constexpr (STAGES == 3) {
                if (ks + 1 < ksteps) step(ks + 1, Int<1>{}, Int<0>{}, mf);
            }
        };
        if constexpr (S::FAST && MT == 2) {
            // One k-loop per count of this wave's fragments that hold rows
            // (a wave-uniform choice per tile; every version has the same
            // barriers): the last row tile of an expert is often mostly empty.
            const int wave_rows = rows_valid - wm * S::kWaveM;
            const int wave_frags =
                __builtin_amdgcn_readfirstlane(wave_rows > 32 ? 2 : wave_rows > 0 ? 1 : 0);
            if (wave_frags == 2) k_loop(Int<2>{});
            else if (wave_frags == 1) k_loop(Int<1>{});
            else k_loop(Int<0>{});
        } else {
            k_loop(Int<MT>{});
        }

        // Epilogue: for the 32 x 32 tile (weight rows n, x rows m), lane l,
        // register r holds n = (l / 32) * 4 + (r / 4) * 8 + r % 4, m = l % 32:
        // registers 4j .. 4j+3 are four consecutive output columns of row m.
        if constexpr (kStagedOut) {
            // Through LDS: each wave writes its bf16 results into the idle
            // weight stages (tile rows 0-63 in b_s0, 64-127 in b_s1, 512 bytes
            // a row, the 16-byte unit u of row r at slot u ^ (r % 32), so the
            // 32 rows of one 8-byte write land in 32 different slots), then
            // every wave stores whole rows, two 512-byte rows per instruction.
            // Stored straight from the MFMA layout, each instruction wrote 16
            // bytes into each of 32 rows.
            lds_barrier();  // every wave is done reading the stages
            __bf16* half = wm == 0 ? b_s0 : b_s1;
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                const int r = mi * 32 + lane % 32;  // row within the half
#pragma unroll
                for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = wn * S::kWaveN + ni * 32 + (lane / 32) * 4 + j * 8;
                        const uint32_t lo =
                            bf16_bits_rne(acc[mi][ni][4 * j]) | (bf16_bits_rne(acc[mi][ni][4 * j + 1]) << 16);
                        const uint32_t hi =
                            bf16_bits_rne(acc[mi][ni][4 * j + 2]) | (bf16_bits_rne(acc[mi][ni][4 * j + 3]) << 16);
                        char* slot = reinterpret_cast<char*>(half) + r * 512 + (((c / 8) ^ (r % 32)) * 16) + (c % 8) * 2;
                        *reinterpret_cast<uint2*>(slot) = make_uint2(lo, hi);
                    }
                }
            }
            lds_barrier();
            constexpr int kRowsPerWave = BM / S::kWaves;
            const int u = lane % 32;
            const __bf16* hb = wave * kRowsPerWave < 64 ? b_s0 : b_s1;  // the wave's rows lie in one half
            u32x4 v[kRowsPerWave / 2];
#pragma unroll
            for (int i = 0; i < kRowsPerWave / 2; ++i) {  // all reads first, then the stores
                const int r = (wave * kRowsPerWave + 2 * i + lane / 32) % 64;
                v[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(hb) + r * 512 +
                                                      ((u ^ (r % 32)) * 16));
            }
#pragma unroll
            for (int i = 0; i < kRowsPerWave / 2; ++i) {
                const int row = wave * kRowsPerWave + 2 * i + lane / 32;  // row of the tile
                if (row < tc.rows) *reinterpret_cast<u32x4*>(y + (tc.row0 + row) * n + tc.col0 + u * 8) = v[i];
            }
        } else {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            const int row = wm * S::kWaveM + mi * 32 + lane % 32;
            if (row >= tc.rows) continue;
            uint16_t* yrow = y + (tc.row0 + row) * n;
#pragma unroll
            for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = tc.col0 + wn * S::kWaveN + ni * 32 + (lane / 32) * 4 + j * 8;
                    const uint32_t lo = bf16_bits_rne(acc[mi][ni][4 * j]) | (bf16_bits_rne(acc[mi][ni][4 * j + 1]) << 16);
                    const uint32_t hi =
                        bf16_bits_rne(acc[mi][ni][4 * j + 2]) | (bf16_bits_rne(acc[mi][ni][4 * j + 3]) << 16);
                    *reinterpret_cast<uint2*>(yrow + col) = make_uint2(lo, hi);
                }
            }
        }
        }
    }
}

template <typename S>
hipError_t launch_gemm_tiles(const GemmArgs& a, int num_cus, hipStream_t stream) {
    // Persistent grid: PER_CU workgroups per compute unit, a multiple of the XCD count.
    int64_t blocks = (int64_t)num_cus * S::PER_CU;
    blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<S>), dim3((unsigned)blocks), dim3(S::kThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(a.x), reinterpret_cast<const u32x4*>(a.w), a.offsets,
                       reinterpret_cast<uint16_t*>(a.y), a.num_experts, a.max_rows, a.n, a.k);
    return hipGetLastError();
}

}  // namespace

// Kernel choice from what the host knows (rows M = max_rows, experts E, n, k).
// The tiled kernel runs at most min(M, E + M / 128) row tiles times n / 256
// column tiles, one workgroup per CU.  At decode sizes the work is streaming
// the experts' weights, and two streaming kernels do it faster:
//  * M <= E (one row per expert on average) and k a multiple of 512 up to
//    8192: the row-streaming kernel (each weight row read whole; two x rows
//    per item).  Against the tiled kernel (DSv3 shape, n 4096, k 7168):
//    N=1 83 -> 70 us (the LDS-staged kernel), N=4 300 -> 261, N=16
//    1008 -> 861, N=32 (M = E) 1598 -> 1483; Mixtral N=4 236 -> 184, Qwen3
//    N=16 106 -> 97.  Two x rows per item stream an expert's weights once per
//    two of its rows, so past M = E it depends on the routing (DSv3 N=64
//    2210 / 2590 against the tiled kernel).
//  * E < M <= 2E and k a multiple of 512 up to 4096: the same kernel with
//    four x rows per item.  Against the LDS-staged kernel: Mixtral N=6 and 8
//    330 -> 311 and 331 -> 312 us, Qwen3 N=24 and 32 139 -> 103 and
//    154 -> 113; at 3E it lost (Mixtral 330 -> 354).
//  * otherwise M <= 4E, or M <= 16E with fewer tiles than CUs: the LDS-staged
//    kernel (16 x rows per item).  Against the tiled kernel: DSv3 N=16
//    1008 / 965 us, N=64 2210 / 2156, N=128 (4E) 2393 / 2400; Mixtral N=8
//    378 / 334, N=16 344 / 336; Qwen3 N=64 183 / 161.
// The row-streaming kernel (2 or 4 x rows per item) and its k range (moe_gemm_skinny.hip).
hipError_t launch_grouped_gemm_rowstream(const GemmArgs& a, int num_cus, int x_rows, hipStream_t stream);
bool gemm_rowstream_fits(int64_t k, int x_rows);

constexpr int64_t kSkinnyMaxRowsPerExpert = 16;
constexpr int64_t kSkinnyAnyRowsPerExpert = 4;

static bool gemm_takes_skinny(int64_t max_rows, int num_experts, int64_t n, int num_cus) {
    const int64_t bound = num_experts + max_rows / 128;
    const int64_t row_tiles = max_rows < bound ? max_rows : bound;
    return max_rows <= kSkinnyAnyRowsPerExpert * num_experts ||
           (max_rows <= kSkinnyMaxRowsPerExpert * num_experts && row_tiles * ((n + 255) / 256) < num_cus);
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, int num_cus, hipStream_t stream) {
    if (a.max_rows <= a.num_experts && gemm_rowstream_fits(a.k, 2)) return launch_grouped_gemm_rowstream(a, num_cus, 2, stream);
    if (a.max_rows <= 2 * (int64_t)a.num_experts && gemm_rowstream_fits(a.k, 4))
        return launch_grouped_gemm_rowstream(a, num_cus, 4, stream);
    if (gemm_takes_skinny(a.max_rows, a.num_experts, a.n, num_cus)) return launch_grouped_gemm_skinny(a, num_cus, stream);
    if (a.n % 256 == 0) return launch_gemm_tiles<GemmShape<128, 256, 2, 4, 3, 1, true>>(a, num_cus, stream);
    return launch_gemm_tiles<GemmShape<128, 128, 2, 2, 2, 2, false>>(a, num_cus, stream);
}

}  // namespace moe
