// Device helpers shared by the ternary linear kernels (gfx950).
#pragma once

#include <atomic>

#include "twd_internal.h"

namespace twd {
namespace kern {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLoadsPerLane = 8;  // 16-byte weight loads in flight per lane

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

__device__ __forceinline__ uint32_t absbits8(const uint4 v) {
    // |bf16| pairs widened to fp32 bit patterns; max over the eight
    const uint32_t m0 = max(v.x << 16 & 0x7FFF0000u, v.x & 0x7FFF0000u);
    const uint32_t m1 = max(v.y << 16 & 0x7FFF0000u, v.y & 0x7FFF0000u);
    const uint32_t m2 = max(v.z << 16 & 0x7FFF0000u, v.z & 0x7FFF0000u);
    const uint32_t m3 = max(v.w << 16 & 0x7FFF0000u, v.w & 0x7FFF0000u);
    return max(max(m0, m1), max(m2, m3));
}

__device__ __forceinline__ uint32_t q8(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}

// Quantize two bf16 pairs (one 32-bit word each) into four int8 lanes.
__device__ __forceinline__ uint32_t quant4(uint32_t lo, uint32_t hi, float inv) {
    return q8(__uint_as_float(lo << 16), inv) |
           q8(__uint_as_float(lo & 0xFFFF0000u), inv) << 8 |
           q8(__uint_as_float(hi << 16), inv) << 16 |
           q8(__uint_as_float(hi & 0xFFFF0000u), inv) << 24;
}

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
