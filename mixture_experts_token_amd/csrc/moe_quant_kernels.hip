// moe_quant_kernels.hip -- quantise while permuting (gfx950): bf16 / f32 token
// rows become fp8 E4M3FN codes with per-token or per-group scales, written to
// every permuted destination of the token.
//
// What is computed: the per-token activation quantisation of vLLM PR #19636
// "[Kernels] MoE refactor" (highlights: per-token quantisation parameters and
// block shapes in the quantisation config), applied to the rows that the
// permute of vLLM PR #14568 ("permute/unpermute kernel for moe optimization",
// PR description) moves.  Per group of consecutive elements (the whole row
// when there is one scale per token): scale = amax / 448 as one float
// division (1 when amax is 0); code = E4M3FN of the float quotient x / scale,
// rounded to nearest with ties to even and saturated at 448; a NaN quotient
// gets the code 0x7F.
//
// The whole row (at most 1024 16-byte vectors) is held in registers -- by one
// wave per token when there are many tokens, by 4 or 16 waves when there are
// few (their amax meets in LDS) -- so the amax is a register, cross-lane and
// at most one LDS reduction, and the row is read exactly once.  The destinations come from the
// inverse index the index permute wrote (-1: not on this rank, not written);
// a token with no destination is not read.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "moe_launch.h"
#include "moe_permute_device.h"
#include "moe_plan.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

// E4M3FN codes of four floats, packed little-endian into one word: each
// value is clamped to [-448, 448] and converted by the gfx950 OCP fp8
// conversion (nearest, ties to even; a bounded probe compared it with a
// software encoder written from the format on every float in [-448, 448]:
// identical).  A NaN gets 0x7F.
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
    const float c0 = fminf(fmaxf(q0, -kE4M3Max), kE4M3Max), c1 = fminf(fmaxf(q1, -kE4M3Max), kE4M3Max);
    const float c2 = fminf(fmaxf(q2, -kE4M3Max), kE4M3Max), c3 = fminf(fmaxf(q3, -kE4M3Max), kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
    const uint32_t nan = (q0 != q0 ? 0x000000FFu : 0u) | (q1 != q1 ? 0x0000FF00u : 0u) |
                         (q2 != q2 ? 0x00FF0000u : 0u) | (q3 != q3 ? 0xFF000000u : 0u);
    return ((uint32_t)w & ~nan) | (0x7F7F7F7Fu & nan);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |x| of one 16-byte vector (NaN never wins a comparison, as in the
// reading of amax: the largest of the comparable magnitudes).
template <bool kBF16>
__device__ __forceinline__ float vec_amax(const u32x4& v) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (kBF16) {
            const float a = fabsf(bf16_lo(v[q])), b = fabsf(bf16_hi(v[q]));
            m = a > m ? a : m;
            m = b > m ? b : m;
        } else {
            const float a = fabsf(__uint_as_float(v[q]));
            m = a > m ? a : m;
        }
    }
    return m;
}

__device__ __forceinline__ float max_xor(float m, int lane_mask) {
    const float o = __shfl_xor(m, lane_mask, 64);
    return o > m ? o : m;
}

// x / scale for bf16 x, giving the code of the correctly rounded quotient
// with one division per scale instead of one per element: the reciprocal r =
// 1 / scale (correctly rounded), q0 = x * r, and the FMA correction step of
// Markstein's division, q = q0 + r * (x - q0 * scale), the sign taken from x
// (an exact zero otherwise loses the sign of -0).  Used for scales in
// [2^-100, 2^126]: an exhaustive host check over every finite bf16 x and every
// scale that a bf16 amax gives (tests/quant_division_check.c) finds the quotient
// bit-identical to the division wherever it can reach a nonzero E4M3 code
// (|x / scale| >= 2^-11) and of the same sign elsewhere; below 2^-100
// (amax < 448 * 2^-100) remainders of subnormal x lose bits, so the division
// stays.  Bf16 inputs only (f32 inputs cannot be checked exhaustively).
struct Bf16Quotient {
    float scale, r;
    bool fast;
    __device__ __forceinline__ explicit Bf16Quotient(float s)
        : scale(s), r(0.0f), fast(s >= 0x1p-100f && s <= 0x1p+126f) {
        if (fast) r = __fdiv_rn(1.0f, s);
    }
    __device__ __forceinline__ float operator()(float x) const {
        if (!fast) return __fdiv_rn(x, scale);
        const float q0 = x * r;
        return copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);
    }
};

// Codes of one 16-byte vector: 8 bf16 -> 8 bytes, or 4 f32 -> 4 bytes (in .x).
template <bool kBF16>
__device__ __forceinline__ u32x2 vec_codes(const u32x4& v, float scale) {
    u32x2 out;
    if constexpr (kBF16) {
        const Bf16Quotient q(scale);
        out.x = e4m3_pack4(q(bf16_lo(v[0])), q(bf16_hi(v[0])), q(bf16_lo(v[1])), q(bf16_hi(v[1])));
        out.y = e4m3_pack4(q(bf16_lo(v[2])), q(bf16_hi(v[2])), q(bf16_lo(v[3])), q(bf16_hi(v[3])));
    } else {
        out.x = e4m3_pack4(__fdiv_rn(__uint_as_float(v[0]), scale), __fdiv_rn(__uint_as_float(v[1]), scale),
                           __fdiv_rn(__uint_as_float(v[2]), scale), __fdiv_rn(__uint_as_float(v[3]), scale));
        out.y = 0u;
    }
    return out;
}

// TPT threads per token (64: one wave; 256 or 1024: several waves whose
// amax meets in LDS), BT = max(TPT, 256) threads per block, BT / TPT tokens
// per block.  Thread gt of a token holds vectors gt, gt + TPT, ...  (U of
// them, U*TPT >= row_vecs); with kPair (bf16, U even) it holds the adjacent
// pairs 2 (gt + TPT p), 2 (gt + TPT p) + 1 instead, so the 16 codes of a pair
// go out as one 16-byte store.  group_vecs: vectors per
// scale group (a power of two <= 64, so a group is an aligned run of lanes of
// one wave; at least 2 with kPair), or 0 for one scale per token.  kAllLocal (no expert map): every token has topk
// destinations, so its row is loaded before anything else is read and the
// check for a rejected id (off[0] < 0: write nothing) follows the loads; with
// a map the destinations are read first and tokens without one are skipped.
template <bool kBF16, int U, int TPT, bool kNTStore, bool kAllLocal, bool kPair>
__global__ __launch_bounds__(TPT > 256 ? TPT : 256) void quant_scatter_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ inv, const int64_t* __restrict__ off,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t num_tokens, int64_t rv, int topk,
    int group_vecs) {
    constexpr int BT = TPT > 256 ? TPT : 256;
    constexpr int TB = BT / TPT;           // tokens per block
    constexpr int WPT = TPT / 64;          // waves per token
    constexpr int kEpv = kBF16 ? 8 : 4;    // elements (and code bytes) per 16-byte input vector
    static_assert(!kPair || (kBF16 && U % 2 == 0), "pairs: bf16 rows, an even number of vectors per thread");
    __shared__ float red_s[WPT > 1 ? WPT : 1];
    if constexpr (!kAllLocal) {
        if (off[0] < 0) return;            // the index permute rejected an id: write nothing
    }
    const int gt = (int)(threadIdx.x % TPT);
    const int64_t rows = num_tokens * topk;
    const int64_t row_bytes = rv * kEpv;   // code bytes per row = H
    const int64_t groups = group_vecs > 0 ? rv / group_vecs : 1;
    const int64_t stride = (int64_t)gridDim.x * TB;
    for (int64_t t = (int64_t)blockIdx.x * TB + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / TPT));
         t < num_tokens; t += stride) {
        const int64_t tt = __builtin_amdgcn_readfirstlane((int)t);
        // Any destination on this rank?  (Wave-uniform reads, scalar path; the
        // same answer for every wave of the token, so the block stays together.)
        if constexpr (!kAllLocal) {
            bool any = false;
            for (int k = 0; k < topk; ++k) {
                const int32_t d = inv[tt * topk + k];
                any |= d >= 0 && (int64_t)d < rows;
            }
            if (!any) continue;
        }
        u32x4 v[U];
        const u32x4* src = x + tt * rv;
        auto vidx = [&](int u) -> int64_t {  // the vector in this thread's slot u
            if constexpr (kPair) return 2 * (gt + (int64_t)TPT * (u / 2)) + u % 2;
            else return gt + (int64_t)TPT * u;
        };
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = vidx(u);
            // a pair's second load reads the lines its first one brought in, so
            // those go through the cache
            if constexpr (kPair) v[u] = idx < rv ? src[idx] : u32x4{0u, 0u, 0u, 0u};
            else v[u] = idx < rv ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (kAllLocal) {
            // the index permute rejected an id: write nothing.  The empty asm
            // keeps this test after the row loads (it cannot be hoisted).
            int64_t off0 = off[0];
            asm volatile("" : "+s"(off0));
            if (off0 < 0) return;
        }
        // Scales: per vector amax, reduced over its group's lanes (or the token).
        float sc[U];
        if (group_vecs == 0) {
            float m = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float a = vec_amax<kBF16>(v[u]);
                m = a > m ? a : m;
            }
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) m = max_xor(m, s);
            if constexpr (WPT > 1) {
                if (gt % 64 == 0) red_s[gt / 64] = m;
                __syncthreads();
#pragma unroll
                for (int w = 0; w < WPT; ++w) m = red_s[w] > m ? red_s[w] : m;
                __syncthreads();  // red_s is rewritten for the next token
            }
            const float scale = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) sc[u] = scale;
        } else {
            if constexpr (kPair) {  // a group is group_vecs / 2 lanes of pairs
#pragma unroll
                for (int u = 0; u < U; u += 2) {
                    float m = vec_amax<kBF16>(v[u]);
                    const float m1 = vec_amax<kBF16>(v[u + 1]);
                    m = m1 > m ? m1 : m;
                    for (int s = 1; s < group_vecs / 2; s <<= 1) m = max_xor(m, s);
                    sc[u] = sc[u + 1] = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float m = vec_amax<kBF16>(v[u]);
                    for (int s = 1; s < group_vecs; s <<= 1) m = max_xor(m, s);
                    sc[u] = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
                }
            }
        }
        u32x2 c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = vec_codes<kBF16>(v[u], sc[u]);
        for (int k = 0; k < topk; ++k) {
            const int32_t d = inv[tt * topk + k];
            if (!(d >= 0 && (int64_t)d < rows)) continue;
            uint8_t* orow = codes + (int64_t)d * row_bytes;
            if constexpr (kPair) {
#pragma unroll
                for (int u = 0; u < U; u += 2) {
                    const int64_t idx = vidx(u);  // even; rv is even, so idx + 1 < rv too
                    if (idx >= rv) continue;
                    u32x4* o = reinterpret_cast<u32x4*>(orow) + idx / 2;
                    const u32x4 cc = {c[u].x, c[u].y, c[u + 1].x, c[u + 1].y};
                    if constexpr (kNTStore) __builtin_nontemporal_store(cc, o);
                    else *o = cc;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (kPair) break;
                const int64_t idx = vidx(u);
                if (idx >= rv) continue;
                if constexpr (kBF16) {
                    u32x2* o = reinterpret_cast<u32x2*>(orow) + idx;
                    if constexpr (kNTStore) __builtin_nontemporal_store(c[u], o);
                    else *o = c[u];
                } else {
                    uint32_t* o = reinterpret_cast<uint32_t*>(orow) + idx;
                    if constexpr (kNTStore) __builtin_nontemporal_store(c[u].x, o);
                    else *o = c[u].x;
                }
            }
            float* srow = scales + (int64_t)d * groups;
            if (group_vecs == 0) {
                if (gt == 0) srow[0] = sc[0];
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t idx = vidx(u);
                    if (idx < rv && idx % group_vecs == 0) srow[idx / group_vecs] = sc[u];
                }
            }
        }
    }
}

template <bool kBF16, int U, int TPT, bool kPair>
hipError_t launch_quant_up(const QuantArgs& a, hipStream_t stream) {
    constexpr int BT = TPT > 256 ? TPT : 256;
    constexpr int64_t TB = BT / TPT;
    const int64_t blocks_needed = (a.num_tokens + TB - 1) / TB;
    const int64_t blocks = blocks_needed < kMaxGridBlocks ? blocks_needed : kMaxGridBlocks;
    // Plain stores for wide fan-out into large outputs, as in the permute row copy.
    const bool plain = a.topk >= 4 && a.num_tokens * a.topk * a.row_vecs * (kBF16 ? 8 : 4) >= (int64_t(32) << 20);
    auto go = [&](auto nt_store, auto all_local) {
        hipLaunchKernelGGL((quant_scatter_kernel<kBF16, U, TPT, decltype(nt_store)::value, decltype(all_local)::value,
                                                 kPair>),
                           dim3((unsigned)blocks), dim3(BT), 0, stream,
                           reinterpret_cast<const u32x4*>(a.hidden_states), a.inv_permuted_idx,
                           a.expert_first_token_offset, a.permuted_codes, a.permuted_scale, a.num_tokens, a.row_vecs,
                           a.topk, a.group_vecs);
    };
    if (plain) {
        if (a.all_local) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    } else {
        if (a.all_local) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    }
    return hipGetLastError();
}

// Adjacent pairs for several waves per token (bf16 rows of an even vector
// count, an even number of vectors per thread, no single-vector scale
// groups): Mixtral-shaped rows, cold in HBM, 21.5 -> 20.6 us per token scale
// and 22.8 -> 20.6 us for groups of 128.  One wave per token keeps single
// vectors: with pairs the Qwen3 shape measured 42.6 -> 44.7 us.
template <bool kBF16, int U, int TPT>
hipError_t launch_quant_ut(const QuantArgs& a, hipStream_t stream) {
    if constexpr (kBF16 && U % 2 == 0 && TPT > 64) {
        if (a.row_vecs % 2 == 0 && a.group_vecs != 1) return launch_quant_up<kBF16, U, TPT, true>(a, stream);
    }
    return launch_quant_up<kBF16, U, TPT, false>(a, stream);
}

// Threads per token: one wave for short rows while tokens alone fill the
// chip; four waves for long rows or fewer tokens (measured faster from 8 KiB
// rows up: shorter serial chains per wave, more waves in flight); sixteen
// when there are very few tokens.
constexpr int64_t kQuantOneWaveMinTokens = 1024;
constexpr int64_t kQuantOneWaveMaxRowVecs = 256;
constexpr int64_t kQuantFourWaveMinTokens = 64;

template <bool kBF16>
hipError_t launch_quant_dtype(const QuantArgs& a, hipStream_t stream) {
    const int64_t rv = a.row_vecs;
    if (a.num_tokens >= kQuantOneWaveMinTokens && rv <= kQuantOneWaveMaxRowVecs) {
        if (rv <= 64) return launch_quant_ut<kBF16, 1, 64>(a, stream);
        if (rv <= 128) return launch_quant_ut<kBF16, 2, 64>(a, stream);
        if (rv <= 192) return launch_quant_ut<kBF16, 3, 64>(a, stream);
        return launch_quant_ut<kBF16, 4, 64>(a, stream);
    }
    if (a.num_tokens >= kQuantFourWaveMinTokens) {
        if (rv <= 256) return launch_quant_ut<kBF16, 1, 256>(a, stream);
        if (rv <= 512) return launch_quant_ut<kBF16, 2, 256>(a, stream);
        if (rv <= 768) return launch_quant_ut<kBF16, 3, 256>(a, stream);
        return launch_quant_ut<kBF16, 4, 256>(a, stream);
    }
    return launch_quant_ut<kBF16, 1, 1024>(a, stream);  // rv <= 1024 (checked on the host)
}

// ----------------------------------------------------------------------------
// Decode sizes (N*topk <= kWaveMaxRows, no expert map): the index permute and
// the quantise-scatter in one kernel of one-wave workgroups, as the wave
// schedule of the plain permute does it.  Grid: chunks of 64 input vectors x
// tokens.  Every wave computes the whole index (wave_index_pass; workgroup
// (0, 0) writes it), then quantises its chunk of its token and stores the
// codes (and scales) at the token's topk destinations.  With one scale per
// token each wave also reads the whole row for the amax (kRowPer vectors per
// lane, from L2 after the first wave); with group scales a chunk holds whole
// groups (a group is at most 64 vectors, aligned).  The arithmetic is the
// quantise-scatter's (vec_amax, max over the group or row, the scale by
// __fdiv_rn, vec_codes).
// ----------------------------------------------------------------------------
template <bool kBF16, typename IdT, int kPer, int kRowPer>
__global__ __launch_bounds__(kWaveSize) void quant_permute_wave_kernel(PermuteArgs a, QuantArgs q, int nbits) {
    constexpr int kEpv = kBF16 ? 8 : 4;  // elements (and code bytes) per 16-byte input vector
    extern __shared__ int smem[];
    const int E = a.num_experts;
    const int K = a.topk;
    const int R = (int)(a.num_tokens * K);
    int* run = smem;
    int* dest_s = run + E;
    const int lane = (int)threadIdx.x;
    const IdT* ids = static_cast<const IdT*>(a.topk_ids);
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;

    // Independent loads first: the ids, this wave's input vector, the row.
    int id[kPer];
    float sc_unused[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int r = j * kWaveSize + lane;
        id[j] = load_id(ids, r < R ? r : R - 1);
    }
    const int64_t rv = q.row_vecs;
    const int t = (int)blockIdx.y;
    const u32x4* src = static_cast<const u32x4*>(q.hidden_states) + (int64_t)t * rv;
    const int64_t idx = (int64_t)blockIdx.x * kWaveSize + lane;  // blockIdx.x < ceil(rv / 64)
    const u32x4 v = __builtin_nontemporal_load(src + (idx < rv ? idx : rv - 1));
    u32x4 row[kRowPer > 0 ? kRowPer : 1];
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
        const int64_t i = (int64_t)j * kWaveSize + lane;
        row[j] = src[i < rv ? i : rv - 1];  // duplicates past the row end do not change a maximum
    }

    if (!wave_index_pass<kPer, false>(E, R, nbits, id, sc_unused, run, dest_s, writer, a.expert_first_token_offset,
                                      a.permuted_idx, a.inv_permuted_idx, nullptr))
        return;  // a rejected id: nothing but the offsets (-1) is written

    float m;
    if constexpr (kRowPer > 0) {  // one scale per token
        m = 0.0f;
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) {
            const float b = vec_amax<kBF16>(row[j]);
            m = b > m ? b : m;
        }
#pragma unroll
        for (int s = 1; s < kWaveSize; s <<= 1) m = max_xor(m, s);
    } else {
        m = idx < rv ? vec_amax<kBF16>(v) : 0.0f;
        for (int s = 1; s < q.group_vecs; s <<= 1) m = max_xor(m, s);
    }
    const float scale = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
    const u32x2 c = vec_codes<kBF16>(v, scale);
    const int64_t row_bytes = rv * kEpv;
    const int64_t groups = q.group_vecs > 0 ? rv / q.group_vecs : 1;
    for (int k = 0; k < K; ++k) {
        const int d = dest_s[t * K + k];
        if (idx < rv) {
            uint8_t* orow = q.permuted_codes + (int64_t)d * row_bytes;
            if constexpr (kBF16) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(orow) + idx);
            else __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(orow) + idx);
            if (kRowPer == 0 && idx % q.group_vecs == 0) q.permuted_scale[(int64_t)d * groups + idx / q.group_vecs] = scale;
        }
        if (kRowPer > 0 && blockIdx.x == 0 && lane == 0) q.permuted_scale[d] = scale;
    }
}

template <bool kBF16, typename IdT, int kPer>
static hipError_t launch_quant_wave_p(const PermuteArgs& a, const QuantArgs& q, const PermutePlan& p,
                                      hipStream_t stream) {
    const dim3 grid((unsigned)((q.row_vecs + kWaveSize - 1) / kWaveSize), (unsigned)a.num_tokens);
    const size_t lds = wave_lds_bytes(a.num_experts, (int)p.rows);
#define MOE_QW(RP) hipLaunchKernelGGL((quant_permute_wave_kernel<kBF16, IdT, kPer, RP>), grid, dim3(kWaveSize), lds, \
                                      stream, a, q, p.nbits)
    if (q.group_vecs > 0) MOE_QW(0);
    else if (q.row_vecs <= 4 * kWaveSize) MOE_QW(4);
    else MOE_QW(16);  // row_vecs <= kQuantMaxRowVecs = 16 * 64
#undef MOE_QW
    return hipGetLastError();
}

template <bool kBF16, typename IdT>
static hipError_t launch_quant_wave_i(const PermuteArgs& a, const QuantArgs& q, const PermutePlan& p,
                                      hipStream_t stream) {
    static_assert(kWaveMaxRows == 2 * kWaveSize && kQuantMaxRowVecs == 16 * kWaveSize,
                  "ids per lane and row vectors per lane of the decode quantising permute");
    if (p.rows <= kWaveSize) return launch_quant_wave_p<kBF16, IdT, 1>(a, q, p, stream);
    return launch_quant_wave_p<kBF16, IdT, 2>(a, q, p, stream);
}

}  // namespace

hipError_t launch_quant_permute_wave(const PermuteArgs& a, const QuantArgs& q, const PermutePlan& p, bool bf16,
                                     hipStream_t stream) {
    if (bf16) return a.ids64 ? launch_quant_wave_i<true, int64_t>(a, q, p, stream)
                             : launch_quant_wave_i<true, int32_t>(a, q, p, stream);
    return a.ids64 ? launch_quant_wave_i<false, int64_t>(a, q, p, stream)
                   : launch_quant_wave_i<false, int32_t>(a, q, p, stream);
}

hipError_t launch_quant_scatter(const QuantArgs& a, bool bf16, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    return bf16 ? launch_quant_dtype<true>(a, stream) : launch_quant_dtype<false>(a, stream);
}

}  // namespace moe
