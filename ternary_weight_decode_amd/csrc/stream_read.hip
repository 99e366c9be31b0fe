// Measurement references.  stream_read: the achievable-bandwidth reference,
// a plain streaming read with the linear kernels' cache policy (16-byte
// non-temporal loads) that fills the chip: one 256-thread workgroup per
// 32 KiB chunk while that needs at most four per compute unit, else one per
// compute unit reading every 256th chunk (the faster form for large buffers:
// 74 us against 77 us with four per unit over 521 MB), each lane keeping
// eight loads in flight.  It reduces what it reads
// to one word and stores it only when it equals a guard value, so the loads
// cannot be removed.  stream_copy: a plain copy of known size, the
// calibration for the HBM byte counters (bytes read = bytes written = size).
#include "twd_internal.h"

namespace twd {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;         // copy kernel: 16-byte words per lane
constexpr int kReadLoads = 8;     // read kernel: loads in flight per lane
constexpr int kCUs = 256;         // compute units of an MI355X
constexpr int kMaxReadGroups = 4 * kCUs;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(
    const uint4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ sink) {
    // workgroup g reads chunks g, g + G, ... of kThreads * kReadLoads words,
    // each chunk contiguous: load u of a lane is word u * kThreads + lane
    constexpr int64_t kChunk = int64_t(kThreads) * kReadLoads;
    uint32_t h = 0;
    for (int64_t c = blockIdx.x; c * kChunk < n16; c += gridDim.x) {
        const int64_t base = c * kChunk + threadIdx.x;
        v4u v[kReadLoads];
#pragma unroll
        for (int u = 0; u < kReadLoads; ++u) {
            const int64_t i = base + int64_t(u) * kThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + i))
                           : v4u{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadLoads; ++u)
            h ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
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
    // one workgroup per chunk, at least one per compute unit; beyond four
    // chunks per unit, one workgroup per unit striding over the chunks
    int64_t grid = (n16 + int64_t(kThreads) * kReadLoads - 1) / (int64_t(kThreads) * kReadLoads);
    grid = grid < kCUs ? kCUs : grid > kMaxReadGroups ? kCUs : grid;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream,
                       static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace twd
