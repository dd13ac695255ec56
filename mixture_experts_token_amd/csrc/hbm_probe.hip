// hbm_probe.hip -- measurement aid for bench.py (not part of the permute ABI).
//
// Plain streaming kernels with the same byte mix as the two operations but
// no index work and contiguous destinations, so bench.py can report, from the
// same run and the same buffers, what this GPU sustains for that mix:
//   fan-out: each of `rows` source rows is read once and written `fanout`
//            times (destination copy c of row t at row c*rows + t);
//   reduce:  `fanin` consecutive source rows are summed (as 32-bit integers,
//            no floating point) into one destination row.
// One wave per chunk of U*64 16-byte vectors of a row (U = 1, 2, 4 or 8 per
// call); non-temporal loads; stores non-temporal or plain.  bench.py times
// every variant and keeps the fastest, so the ceiling is the best plain
// kernel for the mix, not one fixed geometry.
// Library: libhbm_probe.so, C entry points below; sizes are checked on the
// host and every access stays inside [0, rows) x [0, row_vecs).

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int64_t kMaxBlocks = int64_t(1) << 20;

template <bool kNT>
__device__ __forceinline__ void put(u32x4* p, u32x4 v) {
    if constexpr (kNT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <int U, bool kNT>
__global__ __launch_bounds__(256) void fanout_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t rows, int64_t rv, int fanout, int64_t total_waves) {
    const int64_t nch = (rv + U * kWave - 1) / (U * kWave);
    const int64_t items = rows * nch;
    for (int64_t it = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; it < items; it += total_waves) {
        const int64_t t = it / nch;
        const int64_t base = (it - t * nch) * (U * kWave) + threadIdx.x % kWave;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWave;
            v[u] = idx < rv ? __builtin_nontemporal_load(src + t * rv + idx) : u32x4{0u, 0u, 0u, 0u};
        }
        for (int c = 0; c < fanout; ++c) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = base + u * kWave;
                if (idx < rv) put<kNT>(dst + ((int64_t)c * rows + t) * rv + idx, v[u]);
            }
        }
    }
}

template <int U, bool kNT>
__global__ __launch_bounds__(256) void reduce_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t rows, int64_t rv, int fanin, int64_t total_waves) {
    const int64_t nch = (rv + U * kWave - 1) / (U * kWave);
    const int64_t items = rows * nch;
    for (int64_t it = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; it < items; it += total_waves) {
        const int64_t t = it / nch;
        const int64_t base = (it - t * nch) * (U * kWave) + threadIdx.x % kWave;
        u32x4 acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
        for (int c = 0; c < fanin; ++c) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = base + u * kWave;
                if (idx < rv) acc[u] += __builtin_nontemporal_load(src + (t * fanin + c) * rv + idx);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWave;
            if (idx < rv) put<kNT>(dst + t * rv + idx, acc[u]);
        }
    }
}

template <int U>
void launch_u(bool fan, const u32x4* in, u32x4* out, int64_t rows, int64_t rv, int k, bool nt, hipStream_t s) {
    const int64_t items = rows * ((rv + U * kWave - 1) / (U * kWave));
    const int64_t need = (items + 3) / 4;
    const int64_t blocks = need < kMaxBlocks ? need : kMaxBlocks;
    if (fan) {
        if (nt)
            hipLaunchKernelGGL((fanout_kernel<U, true>), dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, rv, k,
                               blocks * 4);
        else
            hipLaunchKernelGGL((fanout_kernel<U, false>), dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, rv,
                               k, blocks * 4);
    } else {
        if (nt)
            hipLaunchKernelGGL((reduce_kernel<U, true>), dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, rv, k,
                               blocks * 4);
        else
            hipLaunchKernelGGL((reduce_kernel<U, false>), dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, rv,
                               k, blocks * 4);
    }
}

int launch(bool fan, const void* src, void* dst, int64_t rows, int64_t row_bytes, int k, int variant,
           void* stream) {
    if (src == nullptr || dst == nullptr || rows < 1 || row_bytes < 16 || row_bytes % 16 || k < 1 || k > 1024 ||
        variant < 0 || variant > 7)
        return 1;
    const int64_t rv = row_bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    const bool nt = (variant & 1) != 0;
    switch (variant >> 1) {
        case 0: launch_u<1>(fan, in, out, rows, rv, k, nt, s); break;
        case 1: launch_u<2>(fan, in, out, rows, rv, k, nt, s); break;
        case 2: launch_u<4>(fan, in, out, rows, rv, k, nt, s); break;
        default: launch_u<8>(fan, in, out, rows, rv, k, nt, s); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" {

// variant in 0..7: bit 0 = non-temporal stores, bits 1-2 select 1, 2, 4 or 8 vectors per lane.
// src: rows x row_bytes; dst: fanout*rows x row_bytes.  Returns 0, 1 (bad argument) or 5 (launch failed).
int hbm_probe_fanout(const void* src, void* dst, int64_t rows, int64_t row_bytes, int fanout, int variant,
                     void* stream) {
    return launch(true, src, dst, rows, row_bytes, fanout, variant, stream);
}

// src: fanin*rows x row_bytes; dst: rows x row_bytes.  Returns 0, 1 (bad argument) or 5 (launch failed).
int hbm_probe_reduce(const void* src, void* dst, int64_t rows, int64_t row_bytes, int fanin, int variant,
                     void* stream) {
    return launch(false, src, dst, rows, row_bytes, fanin, variant, stream);
}

}  // extern "C"
