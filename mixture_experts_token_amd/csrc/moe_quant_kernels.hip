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
// One wave per token: the whole row (at most 1024 16-byte vectors) is held in
// registers, U vectors per lane, so the amax is a register and cross-lane
// reduction and the row is read exactly once.  The destinations come from the
// inverse index the index permute wrote (-1: not on this rank, not written);
// a token with no destination is not read.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_launch.h"
#include "moe_plan.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;
constexpr float kE4M3Max = 448.0f;

// E4M3FN code of q: clamp the magnitude to 448, then round to the nearest
// value with ties to the even fraction.  Below 2^-6 the values are the
// multiples of 2^-9; above, the float's exponent and its fraction rounded to
// three bits (a carry out of the fraction moves to the next exponent).
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const uint32_t u = __float_as_uint(q);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7Fu;  // NaN
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fminf(__uint_as_float(u & 0x7FFFFFFFu), kE4M3Max);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling; rint rounds to nearest even
    } else {
        const uint32_t ua = __float_as_uint(a);
        const uint32_t m = ua & 0x7FFFFFu;
        code = (((ua >> 23) - 120u) << 3) + ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20);
    }
    return sign | code;
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

// Codes of one 16-byte vector: 8 bf16 -> 8 bytes, or 4 f32 -> 4 bytes (in .x).
template <bool kBF16>
__device__ __forceinline__ u32x2 vec_codes(const u32x4& v, float scale) {
    u32x2 out;
    if constexpr (kBF16) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c0 = e4m3_code(__fdiv_rn(bf16_lo(v[2 * h]), scale));
            const uint32_t c1 = e4m3_code(__fdiv_rn(bf16_hi(v[2 * h]), scale));
            const uint32_t c2 = e4m3_code(__fdiv_rn(bf16_lo(v[2 * h + 1]), scale));
            const uint32_t c3 = e4m3_code(__fdiv_rn(bf16_hi(v[2 * h + 1]), scale));
            w[h] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        }
        out.x = w[0];
        out.y = w[1];
    } else {
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = e4m3_code(__fdiv_rn(__uint_as_float(v[q]), scale));
        out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        out.y = 0u;
    }
    return out;
}

// One wave per token t.  U: vectors per lane (U*64 >= row_vecs).  group_vecs:
// vectors per scale group (a power of two <= 64, so a group is an aligned run
// of lanes within one u), or 0 for one scale per token.
template <bool kBF16, int U, bool kNTStore>
__global__ __launch_bounds__(kQuantThreads) void quant_scatter_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ inv, const int64_t* __restrict__ off,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t num_tokens, int64_t rv, int topk,
    int group_vecs, int64_t total_waves) {
    constexpr int kEpv = kBF16 ? 8 : 4;  // elements (and code bytes) per 16-byte input vector
    if (off[0] < 0) return;              // the index permute rejected an id: write nothing
    const int lane = (int)(threadIdx.x % 64);
    const int64_t rows = num_tokens * topk;
    const int64_t row_bytes = rv * kEpv;  // code bytes per row = H
    const int64_t groups = group_vecs > 0 ? rv / group_vecs : 1;
    for (int64_t t = (int64_t)blockIdx.x * (kQuantThreads / 64) + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / 64));
         t < num_tokens; t += total_waves) {
        const int64_t tt = __builtin_amdgcn_readfirstlane((int)t);
        // Any destination on this rank?  (Wave-uniform reads, scalar path.)
        bool any = false;
        for (int k = 0; k < topk; ++k) {
            const int32_t d = inv[tt * topk + k];
            any |= d >= 0 && (int64_t)d < rows;
        }
        if (!any) continue;
        u32x4 v[U];
        const u32x4* src = x + tt * rv;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = lane + 64 * u;
            v[u] = idx < rv ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
        // Scales: per vector amax, reduced over its group's lanes (or the wave).
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
            const float scale = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) sc[u] = scale;
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float m = vec_amax<kBF16>(v[u]);
                for (int s = 1; s < group_vecs; s <<= 1) m = max_xor(m, s);
                sc[u] = m > 0.0f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
            }
        }
        u32x2 c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = vec_codes<kBF16>(v[u], sc[u]);
        for (int k = 0; k < topk; ++k) {
            const int32_t d = inv[tt * topk + k];
            if (!(d >= 0 && (int64_t)d < rows)) continue;
            uint8_t* orow = codes + (int64_t)d * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = lane + 64 * u;
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
                if (lane == 0) srow[0] = sc[0];
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t idx = lane + 64 * u;
                    if (idx < rv && idx % group_vecs == 0) srow[idx / group_vecs] = sc[u];
                }
            }
        }
    }
}

// Vectors per lane: the smallest listed U with U*64 >= row_vecs.
constexpr int kQuantUnrolls[] = {1, 2, 3, 4, 6, 8, 10, 12, 14, 16};

template <bool kBF16, int U>
hipError_t launch_quant_u(const QuantArgs& a, hipStream_t stream) {
    const int64_t waves_needed = a.num_tokens;
    const int64_t per_block = kQuantThreads / 64;
    const int64_t blocks_needed = (waves_needed + per_block - 1) / per_block;
    const int64_t blocks = blocks_needed < kMaxGridBlocks ? blocks_needed : kMaxGridBlocks;
    // Plain stores for wide fan-out into large outputs, as in the permute row copy.
    const bool plain = a.topk >= 4 && a.num_tokens * a.topk * a.row_vecs * (kBF16 ? 8 : 4) >= (int64_t(32) << 20);
    if (plain)
        hipLaunchKernelGGL((quant_scatter_kernel<kBF16, U, false>), dim3((unsigned)blocks), dim3(kQuantThreads), 0,
                           stream, reinterpret_cast<const u32x4*>(a.hidden_states), a.inv_permuted_idx,
                           a.expert_first_token_offset, a.permuted_codes, a.permuted_scale, a.num_tokens, a.row_vecs,
                           a.topk, a.group_vecs, blocks * per_block);
    else
        hipLaunchKernelGGL((quant_scatter_kernel<kBF16, U, true>), dim3((unsigned)blocks), dim3(kQuantThreads), 0,
                           stream, reinterpret_cast<const u32x4*>(a.hidden_states), a.inv_permuted_idx,
                           a.expert_first_token_offset, a.permuted_codes, a.permuted_scale, a.num_tokens, a.row_vecs,
                           a.topk, a.group_vecs, blocks * per_block);
    return hipGetLastError();
}

template <bool kBF16>
hipError_t launch_quant_dtype(const QuantArgs& a, hipStream_t stream) {
    int u = kQuantUnrolls[sizeof(kQuantUnrolls) / sizeof(int) - 1];
    for (int c : kQuantUnrolls)
        if ((int64_t)c * 64 >= a.row_vecs) {
            u = c;
            break;
        }
    switch (u) {
        case 1: return launch_quant_u<kBF16, 1>(a, stream);
        case 2: return launch_quant_u<kBF16, 2>(a, stream);
        case 3: return launch_quant_u<kBF16, 3>(a, stream);
        case 4: return launch_quant_u<kBF16, 4>(a, stream);
        case 6: return launch_quant_u<kBF16, 6>(a, stream);
        case 8: return launch_quant_u<kBF16, 8>(a, stream);
        case 10: return launch_quant_u<kBF16, 10>(a, stream);
        case 12: return launch_quant_u<kBF16, 12>(a, stream);
        case 14: return launch_quant_u<kBF16, 14>(a, stream);
        default: return launch_quant_u<kBF16, 16>(a, stream);
    }
}

}  // namespace

hipError_t launch_quant_scatter(const QuantArgs& a, bool bf16, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    return bf16 ? launch_quant_dtype<true>(a, stream) : launch_quant_dtype<false>(a, stream);
}

}  // namespace moe
