// moe_permute_api.cpp -- the C ABI declared in include/moe_permute.h.
//
// Every argument check runs on the host before anything touches HIP, so a
// rejected call has no side effect and the checks work on a host with no GPU.
// The only HIP calls are the kernel launches, the device queries of
// moe_permute_supported and the grouped GEMM, and (after every check of a
// moe_permute_static_scratch call) the lookup of the static workspace.

#include "moe_permute.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "moe_launch.h"
#include "moe_plan.h"

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;  // int32 indices
constexpr int64_t kMaxRowBytes = int64_t(1) << 40;

int64_t element_bytes(int32_t dtype) {
    switch (dtype) {
        case MOE_DTYPE_F32: return 4;
        case MOE_DTYPE_BF16: return 2;
        case MOE_DTYPE_FP8_E4M3: return 1;
        default: return 0;
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
    const void* p;
    uint64_t bytes;
};

bool overlap(const Span& a, const Span& b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// True if any output overlaps any other output or any input.
bool any_overlap(const Span* outs, int nouts, const Span* ins, int nins) {
    for (int i = 0; i < nouts; ++i) {
        for (int j = i + 1; j < nouts; ++j)
            if (overlap(outs[i], outs[j])) return true;
        for (int j = 0; j < nins; ++j)
            if (overlap(outs[i], ins[j])) return true;
    }
    return false;
}

bool sizes_ok(int64_t num_tokens, int32_t topk, int32_t num_experts) {
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_experts > MOE_MAX_EXPERTS || topk > num_experts)
        return false;
    return num_tokens <= kMaxRows / topk;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

int moe_permute_supported(int device) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess) return 0;
    if (device < 0 || device >= count) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

size_t moe_permute_workspace_size(int64_t max_num_tokens, int32_t topk, int32_t num_experts) {
    if (!sizes_ok(max_num_tokens, topk, num_experts)) return 0;
    return moe::workspace_bound(max_num_tokens, topk, num_experts, 0);
}

size_t moe_permute_local_workspace_size(int64_t max_num_tokens, int32_t topk, int32_t num_experts,
                                        int32_t num_local_experts) {
    if (!sizes_ok(max_num_tokens, topk, num_experts)) return 0;
    if (num_local_experts < 1 || num_local_experts > MOE_MAX_EXPERTS) return 0;
    return moe::workspace_bound(max_num_tokens, topk, num_local_experts, num_experts);
}

}  // extern "C"

namespace {

// Both permute entry points: expert_map == nullptr sorts by expert over
// num_experts buckets; otherwise by local id over num_local_experts buckets.
moe_status_t permute_impl(const void* hidden_states, int32_t dtype, const float* token_scale, const void* topk_ids,
                          int32_t ids_dtype, int64_t num_tokens, int64_t hidden_size, int32_t topk,
                          int32_t num_experts, const int32_t* expert_map, int32_t num_local_experts,
                          void* permuted_hidden_states, float* permuted_scale, int64_t* expert_first_token_offset,
                          int32_t* permuted_idx, int32_t* inv_permuted_idx, void* workspace,
                          size_t workspace_bytes, void* stream, bool static_workspace = false,
                          const moe::QuantArgs* fuse_quant = nullptr, bool quant_bf16 = false,
                          bool* quant_fused = nullptr) {
    const int64_t eb = element_bytes(dtype);
    if (eb == 0) return MOE_ERR_INVALID_ARG;
    if (!sizes_ok(num_tokens, topk, num_experts)) return MOE_ERR_INVALID_ARG;
    const bool mapped = expert_map != nullptr;
    if (mapped && (num_local_experts < 1 || num_local_experts > MOE_MAX_EXPERTS)) return MOE_ERR_INVALID_ARG;
    if (mapped && !aligned(expert_map, 4)) return MOE_ERR_MISALIGNED;
    if (ids_dtype != MOE_DTYPE_INT32 && ids_dtype != MOE_DTYPE_INT64) return MOE_ERR_INVALID_ARG;
    const uint64_t id_bytes = ids_dtype == MOE_DTYPE_INT64 ? 8 : 4;
    const int32_t buckets = mapped ? num_local_experts : num_experts;
    const int map_entries = mapped ? num_experts : 0;
    if (hidden_size < 0 || hidden_size > kMaxRowBytes / eb) return MOE_ERR_INVALID_ARG;
    if (expert_first_token_offset == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned(expert_first_token_offset, 8)) return MOE_ERR_MISALIGNED;
    if ((token_scale == nullptr) != (permuted_scale == nullptr)) return MOE_ERR_INVALID_ARG;
    const int64_t row_bytes = hidden_size * eb;
    if (row_bytes % 16 != 0) return MOE_ERR_MISALIGNED;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (num_tokens == 0) {
        return moe::launch_fill_offsets(expert_first_token_offset, buckets, 0, s) == hipSuccess ? MOE_OK
                                                                                                : MOE_ERR_HIP;
    }
    if (topk_ids == nullptr || permuted_idx == nullptr || inv_permuted_idx == nullptr) return MOE_ERR_INVALID_ARG;
    if (hidden_size > 0 && (hidden_states == nullptr || permuted_hidden_states == nullptr))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(topk_ids, id_bytes) || !aligned(permuted_idx, 4) || !aligned(inv_permuted_idx, 4))
        return MOE_ERR_MISALIGNED;
    if (token_scale != nullptr && (!aligned(token_scale, 4) || !aligned(permuted_scale, 4))) return MOE_ERR_MISALIGNED;
    if (hidden_size > 0 && (!aligned(hidden_states, 16) || !aligned(permuted_hidden_states, 16)))
        return MOE_ERR_MISALIGNED;

    const bool split = moe::split_copy_applies(num_tokens, topk, row_bytes, map_entries);
    moe::PermutePlan plan = moe::plan_permute(num_tokens, topk, buckets, map_entries,
                                              (hidden_size == 0 || split) && token_scale == nullptr);
    plan.split_copy = split;
    if (static_workspace) {
        // the library's static array stands in for the caller's workspace
        if (plan.ws_bytes > moe::kStaticScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
        workspace = nullptr;
    } else {
        if (workspace_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
        if (plan.ws_bytes > 0) {
            if (workspace == nullptr) return MOE_ERR_INVALID_ARG;
            if (!aligned(workspace, 16)) return MOE_ERR_MISALIGNED;
        }
    }

    const uint64_t rows = (uint64_t)plan.rows;
    const bool copy_rows = hidden_size > 0;
    const Span outs[] = {
        {copy_rows ? permuted_hidden_states : nullptr, rows * (uint64_t)row_bytes},
        {permuted_scale, rows * 4},
        {expert_first_token_offset, 8ull * (uint64_t)(buckets + 1)},
        {permuted_idx, rows * 4},
        {inv_permuted_idx, rows * 4},
        {workspace, (uint64_t)plan.ws_bytes},
    };
    const Span ins[] = {
        {copy_rows ? hidden_states : nullptr, (uint64_t)num_tokens * (uint64_t)row_bytes},
        {token_scale, (uint64_t)num_tokens * 4},
        {topk_ids, rows * id_bytes},
        {expert_map, 4ull * (uint64_t)map_entries},
    };
    if (any_overlap(outs, 6, ins, 4)) return MOE_ERR_INVALID_ARG;
    // Every check has passed; only now, and only when the plan uses a
    // workspace, look up this device's static array (once per device).
    if (static_workspace && plan.ws_bytes > 0 && moe::static_scratch_address(&workspace) != hipSuccess)
        return MOE_ERR_HIP;

    moe::PermuteArgs a;
    a.hidden_states = copy_rows ? hidden_states : nullptr;
    a.token_scale = token_scale;
    a.topk_ids = topk_ids;
    a.ids64 = ids_dtype == MOE_DTYPE_INT64;
    a.num_tokens = num_tokens;
    a.row_vecs = row_bytes / 16;
    a.topk = topk;
    a.num_experts = num_experts;
    a.expert_map = expert_map;
    a.num_buckets = buckets;
    a.permuted_hidden_states = copy_rows ? permuted_hidden_states : nullptr;
    a.permuted_scale = permuted_scale;
    a.expert_first_token_offset = expert_first_token_offset;
    a.permuted_idx = permuted_idx;
    a.inv_permuted_idx = inv_permuted_idx;
    if (fuse_quant != nullptr && plan.wave && !mapped) {
        // decode sizes: index permute and quantise-scatter in one kernel
        *quant_fused = true;
        return moe::launch_quant_permute_wave(a, *fuse_quant, plan, quant_bf16, s) == hipSuccess ? MOE_OK
                                                                                                : MOE_ERR_HIP;
    }
    return moe::launch_permute(a, plan, workspace, s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" {

moe_status_t moe_permute(const void* hidden_states, int32_t dtype, const float* token_scale, const void* topk_ids,
                         int32_t topk_ids_dtype, int64_t num_tokens, int64_t hidden_size, int32_t topk,
                         int32_t num_experts, void* permuted_hidden_states, float* permuted_scale,
                         int64_t* expert_first_token_offset, int32_t* permuted_idx, int32_t* inv_permuted_idx,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return permute_impl(hidden_states, dtype, token_scale, topk_ids, topk_ids_dtype, num_tokens, hidden_size, topk,
                        num_experts, nullptr, 0, permuted_hidden_states, permuted_scale, expert_first_token_offset,
                        permuted_idx, inv_permuted_idx, workspace, workspace_bytes, stream);
}

moe_status_t moe_permute_static_scratch(const void* hidden_states, int32_t dtype, const float* token_scale,
                                        const void* topk_ids, int32_t topk_ids_dtype, int64_t num_tokens,
                                        int64_t hidden_size, int32_t topk, int32_t num_experts,
                                        void* permuted_hidden_states, float* permuted_scale,
                                        int64_t* expert_first_token_offset, int32_t* permuted_idx,
                                        int32_t* inv_permuted_idx, void* stream) {
    // moe_permute's checks and plan; the workspace is the device's static
    // array (no allocation: it exists from library load).
    return permute_impl(hidden_states, dtype, token_scale, topk_ids, topk_ids_dtype, num_tokens, hidden_size, topk,
                        num_experts, nullptr, 0, permuted_hidden_states, permuted_scale, expert_first_token_offset,
                        permuted_idx, inv_permuted_idx, nullptr, 0, stream, true);
}

moe_status_t moe_permute_local(const void* hidden_states, int32_t dtype, const float* token_scale,
                               const void* topk_ids, int32_t topk_ids_dtype, int64_t num_tokens,
                               int64_t hidden_size, int32_t topk, int32_t num_experts, const int32_t* expert_map,
                               int32_t num_local_experts,
                               void* permuted_hidden_states, float* permuted_scale,
                               int64_t* expert_first_token_offset, int32_t* permuted_idx,
                               int32_t* inv_permuted_idx, void* workspace, size_t workspace_bytes, void* stream) {
    if (expert_map == nullptr) return MOE_ERR_INVALID_ARG;
    return permute_impl(hidden_states, dtype, token_scale, topk_ids, topk_ids_dtype, num_tokens, hidden_size, topk,
                        num_experts, expert_map, num_local_experts, permuted_hidden_states, permuted_scale,
                        expert_first_token_offset, permuted_idx, inv_permuted_idx, workspace, workspace_bytes,
                        stream);
}

moe_status_t moe_permute_quant_fp8(const void* hidden_states, int32_t dtype, const void* topk_ids,
                                   int32_t topk_ids_dtype, int64_t num_tokens, int64_t hidden_size, int32_t topk,
                                   int32_t num_experts, const int32_t* expert_map, int32_t num_local_experts,
                                   int64_t group_size, uint8_t* permuted_codes, float* permuted_scale,
                                   int64_t* expert_first_token_offset, int32_t* permuted_idx,
                                   int32_t* inv_permuted_idx, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    // Quantiser checks first; permute_impl then checks the rest before it
    // enqueues anything, so a rejected call has no side effect.
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
    const int64_t eb = element_bytes(dtype);
    const int64_t epv = 16 / eb;  // elements per 16-byte vector
    if (hidden_size < 1 || hidden_size > (int64_t)moe::kQuantMaxRowVecs * epv) return MOE_ERR_INVALID_ARG;
    if (hidden_size % epv != 0) return MOE_ERR_MISALIGNED;
    if (expert_map == nullptr && num_local_experts != 0) return MOE_ERR_INVALID_ARG;
    const int64_t g = group_size == 0 ? hidden_size : group_size;
    if (group_size != 0) {
        const bool pow2 = group_size > 0 && (group_size & (group_size - 1)) == 0;
        if (!pow2 || group_size < epv || group_size > 64 * epv || hidden_size % group_size != 0)
            return MOE_ERR_INVALID_ARG;
    }
    if (num_tokens > 0 && (permuted_codes == nullptr || permuted_scale == nullptr || hidden_states == nullptr))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(permuted_codes, 16) || !aligned(permuted_scale, 4) || !aligned(hidden_states, 16))
        return MOE_ERR_MISALIGNED;
    if (num_tokens >= 0 && topk >= 1 && num_tokens <= kMaxRows / topk) {
        const uint64_t rows = (uint64_t)num_tokens * (uint64_t)topk;
        const int32_t buckets = expert_map != nullptr ? num_local_experts : num_experts;
        const uint64_t id_bytes = topk_ids_dtype == MOE_DTYPE_INT64 ? 8 : 4;
        const Span outs[] = {
            {permuted_codes, rows * (uint64_t)hidden_size},
            {permuted_scale, rows * 4ull * (uint64_t)(hidden_size / g)},
        };
        const Span others[] = {
            {hidden_states, (uint64_t)num_tokens * (uint64_t)(hidden_size * eb)},
            {topk_ids, rows * id_bytes},
            {expert_map, 4ull * (uint64_t)(expert_map != nullptr ? num_experts : 0)},
            {expert_first_token_offset, 8ull * (uint64_t)(buckets > 0 ? buckets + 1 : 1)},
            {permuted_idx, rows * 4},
            {inv_permuted_idx, rows * 4},
            {workspace, (uint64_t)workspace_bytes},
        };
        if (any_overlap(outs, 2, others, 7)) return MOE_ERR_INVALID_ARG;
    }
    // Index permute (no rows moved), then the quantise-scatter; at decode sizes
    // (the wave plan, no expert map) one kernel does both.
    moe::QuantArgs q;
    q.hidden_states = hidden_states;
    q.inv_permuted_idx = inv_permuted_idx;
    q.expert_first_token_offset = expert_first_token_offset;
    q.num_tokens = num_tokens;
    q.row_vecs = hidden_size * eb / 16;
    q.topk = topk;
    q.group_vecs = group_size == 0 ? 0 : (int32_t)(group_size / epv);
    q.all_local = expert_map == nullptr;
    q.permuted_codes = permuted_codes;
    q.permuted_scale = permuted_scale;
    bool fused = false;
    const moe_status_t st = permute_impl(nullptr, dtype, nullptr, topk_ids, topk_ids_dtype, num_tokens, 0, topk,
                                         num_experts, expert_map, num_local_experts, nullptr, nullptr,
                                         expert_first_token_offset, permuted_idx, inv_permuted_idx, workspace,
                                         workspace_bytes, stream, false, &q, dtype == MOE_DTYPE_BF16, &fused);
    if (st != MOE_OK || num_tokens == 0 || fused) return st;
    return moe::launch_quant_scatter(q, dtype == MOE_DTYPE_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

moe_status_t moe_grouped_gemm_bf16(const void* x, const void* w, const int64_t* expert_first_token_offset,
                                   int32_t num_experts, int64_t max_rows, int64_t n, int64_t k, void* y,
                                   void* stream) {
    if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS || max_rows < 0) return MOE_ERR_INVALID_ARG;
    if (n < 128 || n % 128 != 0 || k < 64 || k % 64 != 0) return MOE_ERR_INVALID_ARG;
    // k <= 2^20: the kernels address a tile's rows with 32-bit byte offsets (256 rows of 2k bytes)
    if (n > (int64_t(1) << 40) / 2 || k > (int64_t(1) << 20) || max_rows > kMaxRows) return MOE_ERR_INVALID_ARG;
    if (expert_first_token_offset == nullptr || w == nullptr) return MOE_ERR_INVALID_ARG;
    if (max_rows > 0 && (x == nullptr || y == nullptr)) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(expert_first_token_offset, 8))
        return MOE_ERR_MISALIGNED;
    const Span outs[] = {{y, (uint64_t)max_rows * (uint64_t)n * 2}};
    const Span ins[] = {
        {x, (uint64_t)max_rows * (uint64_t)k * 2},
        {w, (uint64_t)num_experts * (uint64_t)n * (uint64_t)k * 2},
        {expert_first_token_offset, 8ull * (uint64_t)(num_experts + 1)},
    };
    if (any_overlap(outs, 1, ins, 3)) return MOE_ERR_INVALID_ARG;
    if (max_rows == 0) return MOE_OK;
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
        return MOE_ERR_HIP;
    moe::GemmArgs g;
    g.x = x;
    g.w = w;
    g.offsets = expert_first_token_offset;
    g.num_experts = num_experts;
    g.max_rows = max_rows;
    g.n = n;
    g.k = k;
    g.y = y;
    return moe::launch_grouped_gemm_bf16(g, cus, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK
                                                                                                 : MOE_ERR_HIP;
}

static moe_status_t unpermute_impl(const void* expanded_output, int32_t dtype, const float* topk_weights,
                                   const int32_t* inv_permuted_idx, int64_t num_tokens, int64_t hidden_size,
                                   int32_t topk, void* output, void* stream, bool few_live) {
    const int64_t eb = element_bytes(dtype);
    if (eb == 0) return MOE_ERR_INVALID_ARG;
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (num_tokens < 0 || topk < 1 || topk > MOE_MAX_EXPERTS || num_tokens > kMaxRows / topk)
        return MOE_ERR_INVALID_ARG;
    if (hidden_size < 1 || hidden_size > kMaxRowBytes / eb) return MOE_ERR_INVALID_ARG;
    const int64_t row_bytes = hidden_size * eb;
    if (row_bytes % 16 != 0) return MOE_ERR_MISALIGNED;
    if (num_tokens == 0) return MOE_OK;
    if (expanded_output == nullptr || topk_weights == nullptr || inv_permuted_idx == nullptr || output == nullptr)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(expanded_output, 16) || !aligned(output, 16) || !aligned(topk_weights, 4) ||
        !aligned(inv_permuted_idx, 4))
        return MOE_ERR_MISALIGNED;
    const uint64_t rows = (uint64_t)num_tokens * (uint64_t)topk;
    const Span outs[] = {{output, (uint64_t)num_tokens * (uint64_t)row_bytes}};
    const Span ins[] = {
        {expanded_output, rows * (uint64_t)row_bytes},
        {topk_weights, rows * 4},
        {inv_permuted_idx, rows * 4},
    };
    if (any_overlap(outs, 1, ins, 3)) return MOE_ERR_INVALID_ARG;

    moe::UnpermuteArgs a;
    a.expanded_output = expanded_output;
    a.topk_weights = topk_weights;
    a.inv_permuted_idx = inv_permuted_idx;
    a.num_tokens = num_tokens;
    a.row_vecs = row_bytes / 16;
    a.topk = topk;
    a.output = output;
    a.few_live = few_live;
    return moe::launch_unpermute(a, dtype == MOE_DTYPE_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

moe_status_t moe_unpermute(const void* expanded_output, int32_t dtype, const float* topk_weights,
                           const int32_t* inv_permuted_idx, int64_t num_tokens, int64_t hidden_size, int32_t topk,
                           void* output, void* stream) {
    return unpermute_impl(expanded_output, dtype, topk_weights, inv_permuted_idx, num_tokens, hidden_size, topk,
                          output, stream, false);
}

moe_status_t moe_unpermute_local(const void* expanded_output, int32_t dtype, const float* topk_weights,
                                 const int32_t* inv_permuted_idx, int64_t num_tokens, int64_t hidden_size,
                                 int32_t topk, void* output, void* stream) {
    return unpermute_impl(expanded_output, dtype, topk_weights, inv_permuted_idx, num_tokens, hidden_size, topk,
                          output, stream, true);
}

}  // extern "C"
