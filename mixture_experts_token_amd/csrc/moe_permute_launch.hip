// moe_permute_launch.hip -- permute schedule dispatch and the offsets fill of an empty call.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_permute_device.h"

namespace moe {

__global__ void fill_offsets_kernel(int64_t* off, int n, int64_t value) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) off[i] = value;
}

hipError_t launch_fill_offsets(int64_t* off, int num_experts, int64_t value, hipStream_t stream) {
    hipLaunchKernelGGL(fill_offsets_kernel, dim3(1), dim3(256), 0, stream, off, num_experts + 1, value);
    return hipGetLastError();
}
hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t stream) {
    const int u = a.topk >= 4 ? choose_unroll(a.row_vecs, kCopyUnrollsWideFanout, 4)
                              : choose_unroll(a.row_vecs, kCopyUnrolls, 8);
    if (p.fused) return launch_permute_fused(a, p, u, stream);
    if (p.coarse) return launch_permute_coarse(a, p, workspace, u, stream);
    return launch_permute_staged(a, p, workspace, u, stream);
}

}  // namespace moe
