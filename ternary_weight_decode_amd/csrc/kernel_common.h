// Device helpers shared by the ternary linear kernels (gfx950).
#pragma once

#include <atomic>

#include "twd_internal.h"

namespace twd {
namespace kern {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLoadsPerLane = 8;  // 16-byte weight loads in flight per lane

// Cache policy of the weight-stream loads: non-temporal.  Each launch reads
// its weights exactly once, so they are marked for early eviction instead
// of pushing the code, kernel arguments and activations of the launches
// that follow out of the caches.
constexpr int kWeightPolicy = 2;  // the nt bit of a gfx950 buffer load

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// A 16-byte weight load through a plain pointer, with the same policy.
__device__ __forceinline__ uint4 load_weight16(const uint4 *p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kPlane0 = 0x03030303u;
constexpr uint32_t kPlane1 = 0x0C0C0C0Cu;  // codes x 4
constexpr uint32_t kPlane2 = 0x30303030u;  // codes x 16
constexpr uint32_t kOnes = 0x01010101u;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c,
                                  false);
}

// Wave-wide reductions: row_shr 1, 2, 4, 8 leaves each 16-lane row's total in
// its lane 15; the four row totals are combined through readlane.  The
// result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ int wave_sum(int v) {
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    v += dpp<0x118>(v);
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) +
           __builtin_amdgcn_readlane(v, 47) + __builtin_amdgcn_readlane(v, 63);
}

// Maximum of non-negative values given as unsigned bit patterns (|x| of a
// float orders like its bits).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = max(v, static_cast<uint32_t>(dpp<0x111>(static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp<0x112>(static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp<0x114>(static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp<0x118>(static_cast<int>(v))));
    const uint32_t a = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 15)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 31)));
    const uint32_t b = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 47)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63)));
    return max(a, b);
}

// Reductions of R independent per-lane values over each 16-lane DPP row at
// once: the total of row i (lanes 16 i .. 16 i + 15) lands in lane 16 i + 15.
// The DPP steps of the R values interleave, so they need no hazard padding.
template <int R>
__device__ __forceinline__ void row_max16(uint32_t (&v)[R]) {
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] = max(v[i], static_cast<uint32_t>(dpp<0x111>(static_cast<int>(v[i]))));
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] = max(v[i], static_cast<uint32_t>(dpp<0x112>(static_cast<int>(v[i]))));
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] = max(v[i], static_cast<uint32_t>(dpp<0x114>(static_cast<int>(v[i]))));
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] = max(v[i], static_cast<uint32_t>(dpp<0x118>(static_cast<int>(v[i]))));
}

template <int R>
__device__ __forceinline__ void row_sum16(int (&v)[R]) {
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] += dpp<0x111>(v[i]);
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] += dpp<0x112>(v[i]);
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] += dpp<0x114>(v[i]);
#pragma unroll
    for (int i = 0; i < R; ++i)
        v[i] += dpp<0x118>(v[i]);
}

// Per-token int8 quantization, q = rint(x * inv), bit-exact with a plain
// fp32 implementation (rint rounds half to even):
//   * the product x * inv is rounded to fp32 on its own (__fmul_rn: never
//     contracted into an fma), then 1.5 * 2^23 is added (__fadd_rn): the
//     sum's ulp is 1, so the FPU's round-to-nearest-even performs rint and
//     the integer lands in the low mantissa bits, whose low byte is q in
//     two's complement;
//   * no clamp is needed: |x| <= a and inv = RN(127 / a) <= (127 / a)(1 +
//     2^-24) give |x * inv| < 127.5, so |q| <= 127 always.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ uint32_t q8bits(float x, float inv) {
    return __float_as_uint(__fadd_rn(__fmul_rn(x, inv), kRoundMagic));
}

// Quantize two bf16 pairs (one 32-bit word each) into four int8 lanes.
__device__ __forceinline__ uint32_t quant4(uint32_t lo, uint32_t hi, float inv) {
    const uint32_t b0 = q8bits(__uint_as_float(lo << 16), inv);
    const uint32_t b1 = q8bits(__uint_as_float(lo & 0xFFFF0000u), inv);
    const uint32_t b2 = q8bits(__uint_as_float(hi << 16), inv);
    const uint32_t b3 = q8bits(__uint_as_float(hi & 0xFFFF0000u), inv);
    // gather the four low bytes (v_perm_b32: selector bytes 0-3 pick the
    // second operand's bytes, 4-7 the first's, 0x0c gives zero)
    const uint32_t lo2 = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);
    const uint32_t hi2 = __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
    return lo2 | hi2;
}

// Running max of |bf16| over pairs packed in 32-bit words: the magnitude of
// a bf16 orders like its low 15 bits, so a packed 16-bit max does it.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 absmax_pair(u16x2 m, uint32_t v) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu));
}

// The fp32 bit pattern of the larger of the two halves.
__device__ __forceinline__ uint32_t absmax_bits(u16x2 m) {
    return static_cast<uint32_t>(m.x > m.y ? m.x : m.y) << 16;
}

// Pin a value where it is computed.  Left alone, the compiler sinks values
// that only the epilogue uses (kernel arguments, the scale division, the
// segment scale) past the weight-load waits, onto the path that runs after
// the last weight lands; an empty asm that reads and rewrites the value keeps
// its computation here, in the shadow of the loads.
__device__ __forceinline__ void settle_v(float &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void settle_v(int &v) { asm volatile("" : "+v"(v)); }
template <typename P>
__device__ __forceinline__ void settle_s(P &p) { asm volatile("" : "+s"(p)); }

__device__ __forceinline__ float row_gamma(const Segments &sg, int n) {
    float g = sg.gamma[0];
#pragma unroll
    for (int s = 1; s < TWD_MAX_SEGMENTS; ++s)
        if (s < sg.nseg && n >= sg.bound[s - 1])
            g = sg.gamma[s];
    return g;
}

// Staged activation rows in LDS are K bytes of data followed by kPad zero bytes:
// lanes whose 64-weight group lies past K (a partial last super chunk) and
// MFMA token columns past M read the zeros, so out-of-range work adds
// nothing and no load needs a per-lane branch.  The extra 16 bytes spread
// consecutive token rows over the LDS banks.
constexpr int kPad = 80;

// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default 64 KiB; once per kernel (not a stream operation, so it is safe
// while a stream is being captured).
inline hipError_t ensure_lds_limit(const void *fn, int lds) {
    constexpr int kSlots = 512;
    constexpr int kMaxLds = 160 * 1024;
    if (lds <= 65536)
        return hipSuccess;
    static std::atomic<const void *> raised[kSlots];
    int slot = 0;
    for (; slot < kSlots; ++slot) {
        const void *v = raised[slot].load(std::memory_order_acquire);
        if (v == fn)
            return hipSuccess;
        if (v == nullptr)
            break;
    }
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e == hipSuccess && slot < kSlots) {
        const void *expected = nullptr;
        raised[slot].compare_exchange_strong(expected, fn);
    }
    return e;
}

}  // namespace kern
}  // namespace twd
