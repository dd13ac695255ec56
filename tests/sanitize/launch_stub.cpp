// Launch layer and HIP runtime for the GPU-less sanitizer build of the C ABI's
// host code (tests/test_sanitize_host.py).
//
// The runtime reports no device.  Each launch function checks that what the
// host side hands it is self-consistent (non-null buffers where the launch
// needs them, a plan whose sizes match the arguments) and counts the call;
// nothing is dereferenced, so fake addresses are fine.  A call that reaches a
// launch with inconsistent arguments aborts, which fails the test.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>

#include "moe_launch.h"
#include "moe_plan.h"

namespace {
std::atomic<long> g_launches{0};

void require(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "launch stub: inconsistent launch arguments: %s\n", what);
        std::abort();
    }
    ++g_launches;
}
}  // namespace

extern "C" {
hipError_t hipGetDeviceCount(int* count) {
    *count = 0;
    return hipSuccess;
}
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipGetDeviceProperties(hipDeviceProp_t*, int) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }

// Launches that reached the stub since the library was loaded.
long moe_stub_launches(void) { return g_launches.load(); }
}

namespace moe {

hipError_t static_scratch_address(void** ptr) {
    *ptr = nullptr;
    return hipErrorNoDevice;
}

hipError_t launch_fill_offsets(int64_t* off, int num_experts, int64_t, hipStream_t) {
    require(off != nullptr && num_experts >= 1 && num_experts <= kMaxExperts, "fill offsets");
    return hipSuccess;
}

hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t) {
    require(a.topk_ids != nullptr && a.permuted_idx != nullptr && a.inv_permuted_idx != nullptr &&
                a.expert_first_token_offset != nullptr && p.rows == a.num_tokens * a.topk &&
                (a.row_vecs == 0 || (a.hidden_states != nullptr && a.permuted_hidden_states != nullptr)) &&
                (p.ws_bytes == 0 || workspace != nullptr),
            "permute");
    return hipSuccess;
}

hipError_t launch_permute_wave(const PermuteArgs&, const PermutePlan&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_permute_fused(const PermuteArgs&, const PermutePlan&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_permute_coarse(const PermuteArgs&, const PermutePlan&, void*, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_permute_staged(const PermuteArgs&, const PermutePlan&, void*, int, hipStream_t) {
    return hipErrorNoDevice;
}

hipError_t launch_permute_rows(const PermuteArgs&, hipStream_t) { return hipErrorNoDevice; }

hipError_t launch_unpermute(const UnpermuteArgs& a, bool, hipStream_t) {
    require(a.expanded_output != nullptr && a.topk_weights != nullptr && a.inv_permuted_idx != nullptr &&
                a.output != nullptr && a.num_tokens > 0 && a.row_vecs > 0,
            "unpermute");
    return hipSuccess;
}

hipError_t launch_quant_permute_wave(const PermuteArgs& a, const QuantArgs& q, const PermutePlan& p, bool,
                                     hipStream_t) {
    require(a.topk_ids != nullptr && a.permuted_idx != nullptr && a.inv_permuted_idx != nullptr &&
                a.expert_first_token_offset != nullptr && p.wave && p.rows == a.num_tokens * a.topk &&
                a.expert_map == nullptr && q.hidden_states != nullptr && q.permuted_codes != nullptr &&
                q.permuted_scale != nullptr && q.row_vecs > 0 && q.row_vecs <= kQuantMaxRowVecs,
            "quant permute wave");
    return hipSuccess;
}

hipError_t launch_quant_scatter(const QuantArgs& a, bool, hipStream_t) {
    require(a.hidden_states != nullptr && a.permuted_codes != nullptr && a.permuted_scale != nullptr &&
                a.row_vecs > 0 && a.row_vecs <= kQuantMaxRowVecs,
            "quant scatter");
    return hipSuccess;
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, int, hipStream_t) {
    require(a.x != nullptr && a.w != nullptr && a.y != nullptr && a.offsets != nullptr, "grouped gemm");
    return hipSuccess;
}

}  // namespace moe
