// moe_gemm_device.h -- device helpers shared by the grouped GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// Exclusive prefix over the threads of a block of kThreads (a multiple of 64)
// of one int64 value each: within each wave by lane shuffles, across the waves
// through LDS (wsum: kThreads / 64 entries) with one barrier.  Every thread of
// the block must call it; total receives the sum over the block.  (The
// work-item lists of the GEMM kernels are this prefix over the per-expert item
// counts; it replaced a log-step scan with two barriers per step.)
template <int kThreads>
__device__ __forceinline__ int64_t block_exclusive_prefix64(int64_t v, int64_t* wsum, int64_t& total) {
    static_assert(kThreads % 64 == 0, "whole waves");
    constexpr int W = kThreads / 64;
    const int lane = (int)(threadIdx.x % 64), w = (int)(threadIdx.x / 64);
    int64_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int64_t before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int64_t c = wsum[i];
        before += i < w ? c : 0;
        total += c;
    }
    return before + x - v;
}

}  // namespace moe
