// Measurement references.  stream_read: the achievable-bandwidth reference,
// a plain streaming read with the linear kernels' load shape and cache
// policy (16-byte non-temporal loads, four in flight per lane, 256-thread
// workgroups); it reduces what it reads
// to one word and stores it only when it equals a guard value, so the loads
// cannot be removed.  stream_copy: a plain copy of known size, the
// calibration for the HBM byte counters (bytes read = bytes written = size).
#include "twd_internal.h"

namespace twd {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(
    const uint4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ sink) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kLoads + threadIdx.x;
    uint4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kThreads;
        if (i < n16) {
            const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + i));
            v[u] = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            v[u] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    uint32_t h = 0;
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
        h ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (h == 0x9E3779B9u)
        sink[threadIdx.x] = h;
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(
    const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kLoads + threadIdx.x;
    uint4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kThreads;
        if (i < n16)
            v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kThreads;
        if (i < n16)
            dst[i] = v[u];
    }
}

}  // namespace

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kThreads * kLoads - 1) / (kThreads * kLoads);
    hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream, static_cast<const uint4 *>(src),
                       static_cast<uint4 *>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kThreads * kLoads - 1) / (kThreads * kLoads);
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream,
                       static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace twd
