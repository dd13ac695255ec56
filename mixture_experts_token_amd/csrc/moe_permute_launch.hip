// moe_permute_launch.hip -- permute schedule dispatch and the offsets fill of an empty call.

#include <hip/hip_runtime.h>

#include <atomic>
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
// Workspace of moe_permute_static_scratch, for callers that cannot allocate.
// One copy per GPU the library runs on, held until the process ends.  Host
// code never uses the name `scratch` as an address (on the host it is a
// stand-in, not device memory): static_scratch_address() takes each device's
// address once with hipGetSymbolAddress and every launch receives that.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kScratchMaxDevices = 64;

hipError_t static_scratch_address(void** ptr) {
    static std::atomic<void*> addr[kScratchMaxDevices];
    *ptr = nullptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // the calling thread's current device is `dev`, so this is dev's copy
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_permute(const PermuteArgs& a, const PermutePlan& p, void* workspace, hipStream_t stream) {
    if (p.split_copy) {
        // the index (and the scales) first, as an index-only call, then the rows
        PermuteArgs ai = a;
        ai.hidden_states = nullptr;
        ai.permuted_hidden_states = nullptr;
        ai.row_vecs = 0;
        PermutePlan pi = p;
        pi.split_copy = false;
        const hipError_t e = launch_permute(ai, pi, workspace, stream);
        if (e != hipSuccess) return e;
        return launch_permute_rows(a, stream);
    }
    const int u = a.topk >= 4 ? choose_unroll(a.row_vecs, kCopyUnrollsWideFanout, 4)
                              : choose_unroll(a.row_vecs, kCopyUnrolls, 8);
    if (p.wave) return launch_permute_wave(a, p, u, stream);
    if (p.fused) return launch_permute_fused(a, p, u, stream);
    if (p.coarse) return launch_permute_coarse(a, p, workspace, u, stream);
    return launch_permute_staged(a, p, workspace, u, stream);
}

}  // namespace moe
