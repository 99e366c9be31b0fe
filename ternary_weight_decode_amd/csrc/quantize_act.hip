// Per-token absmax int8 activation quantizer for gfx950 (BitMTP page,
// ai.info AI summary, "Main Findings": W2A8 uses 8-bit activations).  One
// workgroup per token row: every 16-byte chunk of the row is loaded at once
// (up to 16384 elements stay in registers), a max-reduction of |x| (packed
// 16-bit max, DPP, one LDS exchange), one correctly rounded fp32 division for
// 127/a, then q = rint(x * inv) written eight at a time.  The rounding
// arithmetic is shared with the fused linear kernels, so both produce the
// same bytes.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

constexpr int kQThreads = 256;
constexpr int kHold = 8;  // chunks of 8 elements held per thread

__global__ __launch_bounds__(kQThreads) void quantize_act_kernel(
    const uint16_t *__restrict__ x, int K, int8_t *__restrict__ xq,
    float *__restrict__ xscale) {
    __shared__ uint32_t wave_max[kQThreads / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + static_cast<int64_t>(m) * K);
    uint2 *out = reinterpret_cast<uint2 *>(xq + static_cast<int64_t>(m) * K);
    const int n8 = K / 8;

    uint4 v[kHold];
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int c = tid + kQThreads * j;
        v[j] = c < n8 ? row[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    u16x2 am2 = {0, 0};
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        am2 = absmax_pair(am2, v[j].x);
        am2 = absmax_pair(am2, v[j].y);
        am2 = absmax_pair(am2, v[j].z);
        am2 = absmax_pair(am2, v[j].w);
    }
    // rows longer than the held part (K > 16384)
    for (int c = tid + kQThreads * kHold; c < n8; c += kQThreads) {
        const uint4 w = row[c];
        am2 = absmax_pair(am2, w.x);
        am2 = absmax_pair(am2, w.y);
        am2 = absmax_pair(am2, w.z);
        am2 = absmax_pair(am2, w.w);
    }
    const uint32_t wm = wave_umax(absmax_bits(am2));
    if ((tid & 63) == 0)
        wave_max[tid >> 6] = wm;
    __syncthreads();
    const uint32_t ab = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    const float a = __uint_as_float(ab);
    // correctly rounded fp32 division (build flag); all-zero row -> zeros
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int c = tid + kQThreads * j;
        if (c < n8)
            out[c] = make_uint2(quant4(v[j].x, v[j].y, inv), quant4(v[j].z, v[j].w, inv));
    }
    for (int c = tid + kQThreads * kHold; c < n8; c += kQThreads) {
        const uint4 w = row[c];
        out[c] = make_uint2(quant4(w.x, w.y, inv), quant4(w.z, w.w, inv));
    }
    if (tid == 0)
        xscale[m] = a / 127.0f;
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int M, int K, int8_t *xq,
                               float *xscale, hipStream_t stream) {
    hipLaunchKernelGGL(quantize_act_kernel, dim3(M), dim3(kQThreads), 0, stream,
                       x, K, xq, xscale);
    return hipGetLastError();
}

}  // namespace twd
