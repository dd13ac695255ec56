// moe_launch.h -- internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_plan.h"

namespace moe {

struct PermuteArgs {
    const void* hidden_states;      // [N, row_vecs * 16 bytes] or null when row_vecs == 0
    const float* token_scale;       // [N] or null
    const void* topk_ids;           // [N, topk] int32, or int64 when ids64
    bool ids64;
    int64_t num_tokens;
    int64_t row_vecs;               // row length in 16-byte vectors (0: indices only)
    int32_t topk;
    int32_t num_experts;            // ids are valid in [0, num_experts)
    const int32_t* expert_map;      // [num_experts] local id or -1, or null (every expert is local)
    int32_t num_buckets;            // sort keys: num_experts, or the local expert count with a map
    void* permuted_hidden_states;   // [N*topk, row_vecs * 16 bytes]
    float* permuted_scale;          // [N*topk] or null
    int64_t* expert_first_token_offset;  // [num_buckets + 1]
    int32_t* permuted_idx;          // [N*topk]
    int32_t* inv_permuted_idx;      // [N*topk]
};

struct UnpermuteArgs {
    const void* expanded_output;    // [N*topk, row_vecs * 16 bytes]
    const float* topk_weights;      // [N, topk]
    const int32_t* inv_permuted_idx;  // [N*topk]
    int64_t num_tokens;
    int64_t row_vecs;
    int32_t topk;
    void* output;                   // [N, row_vecs * 16 bytes]
    bool few_live;                  // most slots are expected to be -1 (an expert split): no occupancy cap
};

struct QuantArgs {
    const void* hidden_states;      // [N, row_vecs * 16 bytes] bf16 or f32
    const int32_t* inv_permuted_idx;  // [N*topk], -1 for rows with no destination
    const int64_t* expert_first_token_offset;  // entry 0 is -1 when the index permute failed
    int64_t num_tokens;
    int64_t row_vecs;               // input row length in 16-byte vectors (<= kQuantMaxRowVecs)
    int32_t topk;
    int32_t group_vecs;             // 16-byte input vectors per scale group; 0: one scale per token
    bool all_local;                 // no expert map: every token has topk destinations
    uint8_t* permuted_codes;        // [N*topk, H] E4M3FN
    float* permuted_scale;          // [N*topk, groups]
};

struct GemmArgs {
    const void* x;                  // [max_rows, k] bf16 (permuted rows)
    const void* w;                  // [num_experts, n, k] bf16
    const int64_t* offsets;         // [num_experts + 1] (device)
    int32_t num_experts;
    int64_t max_rows;
    int64_t n;                      // multiple of 128
    int64_t k;                      // multiple of 64
    void* y;                        // [max_rows, n] bf16
};

hipError_t launch_fill_offsets(int64_t* off, int num_experts, int64_t value, hipStream_t stream);
hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, int num_cus, hipStream_t stream);
// The grouped GEMM for experts with few rows each (called by launch_grouped_gemm_bf16).
hipError_t launch_grouped_gemm_skinny(const GemmArgs& a, int num_cus, hipStream_t stream);
hipError_t launch_quant_scatter(const QuantArgs& a, bool bf16, hipStream_t stream);
// Decode sizes (the wave plan, no expert map): index permute and quantise-scatter in one kernel.
hipError_t launch_quant_permute_wave(const PermuteArgs& a, const QuantArgs& q, const PermutePlan& p, bool bf16,
                                     hipStream_t stream);
hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t stream);
// Device address of the current device's static workspace (kStaticScratchBytes).
hipError_t static_scratch_address(void** ptr);
// One schedule each (u: 16-byte vectors per lane in the row copy).
hipError_t launch_permute_wave(const PermuteArgs& a, const PermutePlan& p, int u, hipStream_t stream);
hipError_t launch_permute_fused(const PermuteArgs& a, const PermutePlan& p, int u, hipStream_t stream);
hipError_t launch_permute_coarse(const PermuteArgs& a, const PermutePlan& p, void* workspace, int u,
                                 hipStream_t stream);
hipError_t launch_permute_staged(const PermuteArgs& a, const PermutePlan& p, void* workspace, int u,
                                 hipStream_t stream);
// Row copy of the split schedule; reads the inverse index and offsets the index pass wrote.
hipError_t launch_permute_rows(const PermuteArgs& a, hipStream_t stream);
hipError_t launch_unpermute(const UnpermuteArgs& a, bool bf16, hipStream_t stream);

}  // namespace moe
