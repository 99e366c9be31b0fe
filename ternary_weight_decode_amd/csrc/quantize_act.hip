// Per-token absmax int8 activation quantizer for gfx950 (BitMTP page,
// ai.info AI summary, "Main Findings": W2A8 uses 8-bit activations).  One
// workgroup per token row: a max-reduction of |x| over the row, one
// correctly rounded fp32 division for 127/a, then q = clamp(rint(x * inv))
// written eight at a time.
#include "twd_internal.h"

namespace twd {
namespace {

constexpr int kThreads = 256;

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline float absmax8(const uint4 v) {
    float a = fabsf(bf16_lo(v.x));
    a = fmaxf(a, fabsf(bf16_hi(v.x)));
    a = fmaxf(a, fabsf(bf16_lo(v.y)));
    a = fmaxf(a, fabsf(bf16_hi(v.y)));
    a = fmaxf(a, fabsf(bf16_lo(v.z)));
    a = fmaxf(a, fabsf(bf16_hi(v.z)));
    a = fmaxf(a, fabsf(bf16_lo(v.w)));
    a = fmaxf(a, fabsf(bf16_hi(v.w)));
    return a;
}

__device__ inline uint32_t q8(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}

__device__ inline uint32_t quant4(uint32_t lo, uint32_t hi, float inv) {
    return q8(bf16_lo(lo), inv) | q8(bf16_hi(lo), inv) << 8 |
           q8(bf16_lo(hi), inv) << 16 | q8(bf16_hi(hi), inv) << 24;
}

__global__ __launch_bounds__(kThreads) void quantize_act_kernel(
    const uint16_t *__restrict__ x, int K, int8_t *__restrict__ xq,
    float *__restrict__ xscale) {
    __shared__ float wave_max[kThreads / 64];
    const int m = blockIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + static_cast<int64_t>(m) * K);
    uint2 *out = reinterpret_cast<uint2 *>(xq + static_cast<int64_t>(m) * K);
    const int n8 = K / 8;

    float a = 0.0f;
    for (int i = threadIdx.x; i < n8; i += kThreads)
        a = fmaxf(a, absmax8(row[i]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));

    if (a == 0.0f) {
        for (int i = threadIdx.x; i < n8; i += kThreads)
            out[i] = make_uint2(0u, 0u);
        if (threadIdx.x == 0)
            xscale[m] = 0.0f;
        return;
    }
    // IEEE division (the library is built with correctly rounded fp32
    // division), then one rounded multiply per element.
    const float inv = 127.0f / a;
    for (int i = threadIdx.x; i < n8; i += kThreads) {
        const uint4 v = row[i];
        out[i] = make_uint2(quant4(v.x, v.y, inv), quant4(v.z, v.w, inv));
    }
    if (threadIdx.x == 0)
        xscale[m] = a / 127.0f;
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int M, int K, int8_t *xq,
                               float *xscale, hipStream_t stream) {
    hipLaunchKernelGGL(quantize_act_kernel, dim3(M), dim3(kThreads), 0, stream,
                       x, K, xq, xscale);
    return hipGetLastError();
}

}  // namespace twd
