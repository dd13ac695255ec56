// hbm_probe.hip -- measurement aid for bench.py (not part of the permute ABI).
//
// Plain streaming kernels with the same byte mix as the two operations but
// no index work and contiguous destinations, so bench.py can report, from the
// same run and the same buffers, what this GPU sustains for that mix:
//   fan-out: each of `rows` source rows is read once and written `fanout`
//            times (destination copy c of row t at row c*rows + t);
//   reduce:  `fanin` consecutive source rows are summed (as 32-bit integers,
//            no floating point) into one destination row;
//   read:    every source row is read and nothing is written (the lanes fold
//            what they read into a value stored only if it equals a constant
//            no input here produces, so the loads cannot be dropped);
//   write:   every destination row is written and nothing is read;
//   fan-out from a few rows: the fan-out's writes, with source row
//            t % source_rows (a set small enough to stay in a cache), or with
//            no reads at all (source_rows 0: a position pattern is written).
// The read and write kernels split a mix into its directions: bench.py times
// each direction of an operation's bytes alone beside the mixed kernels.
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
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ sink,
                                                   int64_t rows, int64_t rv, int64_t total_waves) {
    const int64_t nch = (rv + U * kWave - 1) / (U * kWave);
    const int64_t items = rows * nch;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t it = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; it < items; it += total_waves) {
        const int64_t t = it / nch;
        const int64_t base = (it - t * nch) * (U * kWave) + threadIdx.x % kWave;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWave;
            v[u] = idx < rv ? __builtin_nontemporal_load(src + t * rv + idx) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0xF39CC060u && acc.w == 0x5CEDC834u)
        sink[threadIdx.x] = acc;  // never taken for real data; keeps the loads
}

template <int U, bool kNT>
__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ dst, int64_t rows, int64_t rv,
                                                    int64_t total_waves) {
    const int64_t nch = (rv + U * kWave - 1) / (U * kWave);
    const int64_t items = rows * nch;
    for (int64_t it = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; it < items; it += total_waves) {
        const int64_t t = it / nch;
        const int64_t base = (it - t * nch) * (U * kWave) + threadIdx.x % kWave;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWave;
            const uint32_t p = (uint32_t)(t * rv + idx);
            if (idx < rv) put<kNT>(dst + t * rv + idx, u32x4{p, p, p, p});
        }
    }
}

// Plain stores, two vectors per lane (the fastest fan-out variant at the DSv3 shape).
__global__ __launch_bounds__(256) void fanout_source_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t rows, int64_t rv, int fanout, int64_t source_rows,
                                                            int64_t total_waves) {
    constexpr int U = 2;
    const int64_t nch = (rv + U * kWave - 1) / (U * kWave);
    const int64_t items = rows * nch;
    for (int64_t it = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; it < items; it += total_waves) {
        const int64_t t = it / nch;
        const int64_t base = (it - t * nch) * (U * kWave) + threadIdx.x % kWave;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * kWave;
            if (source_rows == 0) {
                const uint32_t p = (uint32_t)(t * rv + idx);
                v[u] = u32x4{p, p ^ 1u, p ^ 2u, p ^ 3u};
            } else {
                v[u] = idx < rv ? __builtin_nontemporal_load(src + (t % source_rows) * rv + idx)
                                : u32x4{0u, 0u, 0u, 0u};
            }
        }
        for (int c = 0; c < fanout; ++c) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t idx = base + u * kWave;
                if (idx < rv) put<false>(dst + ((int64_t)c * rows + t) * rv + idx, v[u]);
            }
        }
    }
}

template <int U>
int64_t probe_blocks(int64_t rows, int64_t rv) {
    const int64_t items = rows * ((rv + U * kWave - 1) / (U * kWave));
    const int64_t need = (items + 3) / 4;
    return need < kMaxBlocks ? need : kMaxBlocks;
}

template <int U>
void launch_dir(bool read, const u32x4* in, u32x4* out, int64_t rows, int64_t rv, bool nt, hipStream_t s) {
    const int64_t blocks = probe_blocks<U>(rows, rv);
    if (read)
        hipLaunchKernelGGL((read_kernel<U>), dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, rv, blocks * 4);
    else if (nt)
        hipLaunchKernelGGL((write_kernel<U, true>), dim3((unsigned)blocks), dim3(256), 0, s, out, rows, rv,
                           blocks * 4);
    else
        hipLaunchKernelGGL((write_kernel<U, false>), dim3((unsigned)blocks), dim3(256), 0, s, out, rows, rv,
                           blocks * 4);
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

// Read-only (read) or write-only (!read) pass; variant as for launch.
int launch_direction(bool read, const void* src, void* dst, int64_t rows, int64_t row_bytes, int variant,
                     void* stream) {
    if ((read && src == nullptr) || dst == nullptr || rows < 1 || row_bytes < 16 || row_bytes % 16 || variant < 0 ||
        variant > 7)
        return 1;
    const int64_t rv = row_bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    const bool nt = (variant & 1) != 0;
    switch (variant >> 1) {
        case 0: launch_dir<1>(read, in, out, rows, rv, nt, s); break;
        case 1: launch_dir<2>(read, in, out, rows, rv, nt, s); break;
        case 2: launch_dir<4>(read, in, out, rows, rv, nt, s); break;
        default: launch_dir<8>(read, in, out, rows, rv, nt, s); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" {

// src: rows x row_bytes, all read; sink: at least 256 x 16 bytes (written only
// for an input no real data produces).  variant as below (bit 0 ignored).
int hbm_probe_read(const void* src, void* sink, int64_t rows, int64_t row_bytes, int variant, void* stream) {
    return launch_direction(true, src, sink, rows, row_bytes, variant, stream);
}

// dst: rows x row_bytes, all written (a position pattern).
int hbm_probe_write(void* dst, int64_t rows, int64_t row_bytes, int variant, void* stream) {
    return launch_direction(false, nullptr, dst, rows, row_bytes, variant, stream);
}

// The fan-out's writes (dst: fanout*rows x row_bytes) from source rows
// t % source_rows of src (source_rows x row_bytes), or from no source
// (source_rows 0, src unused).  Returns 0, 1 (bad argument) or 5.
int hbm_probe_fanout_source(const void* src, void* dst, int64_t rows, int64_t row_bytes, int fanout,
                            int64_t source_rows, void* stream) {
    if (dst == nullptr || rows < 1 || row_bytes < 16 || row_bytes % 16 || fanout < 1 || fanout > 1024 ||
        source_rows < 0 || (source_rows > 0 && src == nullptr))
        return 1;
    const int64_t rv = row_bytes / 16;
    const int64_t blocks = probe_blocks<2>(rows, rv);
    hipLaunchKernelGGL(fanout_source_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), rows, rv, fanout, source_rows,
                       blocks * 4);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}


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
