// Host-side weight preparation: absmean ternarization and the 2-bit packed
// format (BitMTP page, ai.info AI summary: ternary BitNet b1.58 weights in
// "What This Paper Is About"; packed W2A8 execution in "Methodology in Plain
// English").  These run once when weights are loaded, never per token.
#include <cmath>
#include <cstring>

#include "twd_internal.h"

namespace {

// 16-weight word: element e = 4*j + b sits at bit 8*b + 2*j.
inline int field_shift(int e) { return 8 * (e & 3) + 2 * (e >> 2); }

// fp32 -> OCP E4M3 code by rounding the fp32 bit pattern: nearest, ties to
// even.  Returns false when the value rounds beyond the largest finite code
// (448) or is not finite.
bool e4m3_from_bits(uint32_t u, uint8_t *code) {
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x7F800000u)
        return false;
    const int e32 = static_cast<int>(a >> 23) - 127;
    uint32_t c;
    if (e32 >= -6) {
        // keep the exponent and 3 mantissa bits, round on the other 20
        uint32_t keep = a >> 20;
        const uint32_t rest = a & 0xFFFFFu;
        if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u)))
            ++keep;  // a carry moves into the exponent, as it should
        c = keep - (120u << 3);  // rebias 127 -> 7
        if (c > 0x7Eu)
            return false;
    } else if (a < 0x00800000u) {
        c = 0;  // fp32 subnormal: far below half the smallest E4M3 step
    } else {
        // subnormal E4M3: m = value / 2^-9, with value = sig 2^(e32 - 23)
        const uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;
        const int shift = 14 - e32;  // >= 21
        if (shift > 25) {
            c = 0;
        } else {
            uint32_t m = sig >> shift;
            const uint32_t rest = sig & ((1u << shift) - 1u);
            const uint32_t half = 1u << (shift - 1);
            if (rest > half || (rest == half && (m & 1u)))
                ++m;  // m == 8 is the smallest normal code, 0x08
            c = m;
        }
    }
    *code = static_cast<uint8_t>(sign | c);
    return true;
}

}  // namespace

extern "C" twd_status twd_ternarize_absmean(const float *W, int64_t N,
                                            int64_t K, int8_t *codes,
                                            float *gamma) {
    using twd::set_error;
    if (!W || !codes || !gamma)
        return set_error(TWD_ERR_INVALID_ARG, "ternarize: null pointer");
    if (N < 0 || K < 0)
        return set_error(TWD_ERR_INVALID_ARG, "ternarize: negative size");
    const int64_t count = N * K;
    // Mean of |W|: one double accumulator, row-major order, then a single
    // rounding to fp32, so every implementation following the same order
    // gets the same scale bits.
    double total = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        const float v = W[i];
        if (!std::isfinite(v))
            return set_error(TWD_ERR_INVALID_ARG,
                             "ternarize: non-finite weight at %lld",
                             (long long)i);
        total += std::fabs(static_cast<double>(v));
    }
    const float g = count ? static_cast<float>(total / static_cast<double>(count))
                          : 0.0f;
    *gamma = g;
    if (g == 0.0f) {
        std::memset(codes, 0, static_cast<size_t>(count));
        return TWD_OK;
    }
    for (int64_t i = 0; i < count; ++i) {
        // fp32 quotient, nearest-even rounding (the default FP environment),
        // then clip to the ternary range.
        const float r = std::nearbyint(W[i] / g);
        codes[i] = r >= 1.0f ? 1 : (r <= -1.0f ? -1 : 0);
    }
    return TWD_OK;
}

extern "C" twd_status twd_pack_ternary(const int8_t *codes, int64_t N,
                                       int64_t K, uint8_t *packed) {
    using twd::set_error;
    if (!codes || !packed)
        return set_error(TWD_ERR_INVALID_ARG, "pack: null pointer");
    if (N < 0 || K < 0 || K % 16 != 0)
        return set_error(TWD_ERR_INVALID_ARG,
                         "pack: need N >= 0 and K >= 0 with K %% 16 == 0");
    const int64_t words_per_row = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *row = codes + n * K;
        uint8_t *out = packed + n * (K / 4);
        for (int64_t wi = 0; wi < words_per_row; ++wi) {
            uint32_t word = 0;
            for (int e = 0; e < 16; ++e) {
                const int t = row[16 * wi + e];
                if (t < -1 || t > 1)
                    return set_error(TWD_ERR_BAD_CODE,
                                     "pack: code %d at row %lld col %lld", t,
                                     (long long)n, (long long)(16 * wi + e));
                word |= static_cast<uint32_t>(t + 1) << field_shift(e);
            }
            // little-endian byte order regardless of the host
            out[4 * wi + 0] = static_cast<uint8_t>(word);
            out[4 * wi + 1] = static_cast<uint8_t>(word >> 8);
            out[4 * wi + 2] = static_cast<uint8_t>(word >> 16);
            out[4 * wi + 3] = static_cast<uint8_t>(word >> 24);
        }
    }
    return TWD_OK;
}

extern "C" twd_status twd_unpack_ternary(const uint8_t *packed, int64_t N,
                                         int64_t K, int8_t *codes) {
    using twd::set_error;
    if (!codes || !packed)
        return set_error(TWD_ERR_INVALID_ARG, "unpack: null pointer");
    if (N < 0 || K < 0 || K % 16 != 0)
        return set_error(TWD_ERR_INVALID_ARG,
                         "unpack: need N >= 0 and K >= 0 with K %% 16 == 0");
    const int64_t words_per_row = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *in = packed + n * (K / 4);
        int8_t *row = codes + n * K;
        for (int64_t wi = 0; wi < words_per_row; ++wi) {
            const uint32_t word = static_cast<uint32_t>(in[4 * wi]) |
                                  static_cast<uint32_t>(in[4 * wi + 1]) << 8 |
                                  static_cast<uint32_t>(in[4 * wi + 2]) << 16 |
                                  static_cast<uint32_t>(in[4 * wi + 3]) << 24;
            for (int e = 0; e < 16; ++e) {
                const uint32_t c = (word >> field_shift(e)) & 3u;
                if (c == 3u)
                    return set_error(TWD_ERR_BAD_CODE,
                                     "unpack: invalid code 3 at row %lld col "
                                     "%lld",
                                     (long long)n, (long long)(16 * wi + e));
                row[16 * wi + e] = static_cast<int8_t>(static_cast<int>(c) - 1);
            }
        }
    }
    return TWD_OK;
}

// Per-output-row FP8 quantization for the fast projection: inv = 448 /
// max|row| (fp32 division), code = E4M3(w * inv) (fp32 multiply, nearest
// even), scale = max|row| / 448; an all-zero row gives zero codes and scale 0.
extern "C" twd_status twd_quantize_fp8_rows(const float *W, int64_t N, int64_t K,
                                            uint8_t *codes, float *scale) {
    using twd::set_error;
    if (!W || !codes || !scale)
        return set_error(TWD_ERR_INVALID_ARG, "quantize_fp8_rows: null pointer");
    if (N < 0 || K < 0)
        return set_error(TWD_ERR_INVALID_ARG, "quantize_fp8_rows: negative size");
    for (int64_t n = 0; n < N; ++n) {
        const float *row = W + n * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!std::isfinite(row[k]))
                return set_error(TWD_ERR_INVALID_ARG,
                                 "quantize_fp8_rows: non-finite weight at row %lld",
                                 (long long)n);
            a = std::fmax(a, std::fabs(row[k]));
        }
        uint8_t *out = codes + n * K;
        if (a == 0.0f) {
            std::memset(out, 0, static_cast<size_t>(K));
            scale[n] = 0.0f;
            continue;
        }
        const float inv = 448.0f / a;
        for (int64_t k = 0; k < K; ++k) {
            const float p = row[k] * inv;
            uint32_t bits;
            std::memcpy(&bits, &p, sizeof bits);
            if (!e4m3_from_bits(bits, &out[k]))
                return set_error(TWD_ERR_INVALID_ARG,
                                 "quantize_fp8_rows: value beyond E4M3 at row %lld",
                                 (long long)n);
        }
        scale[n] = a / 448.0f;
    }
    return TWD_OK;
}

// The multi-projection sweep's tiled weight layout: 16-row tiles, each a
// contiguous run of one 1 KiB block per 256-wide K slice; block u of tile t
// holds, at lane l = 16 g + r (16 bytes each), the packed bytes 64 u + 16 g
// .. + 15 of row 16 t + r.  Zeros pad rows past N and bytes past K / 4 (a
// zero byte is code 0 in every field, which the kernels read as "contributes
// nothing": their sums run over c = t + 1 and subtract the activation sum
// over the real K only).
extern "C" int64_t twd_sweep_tiled_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % 64 != 0)
        return -1;
    return ((N + 15) / 16) * ((K + 255) / 256) * 1024;
}

extern "C" twd_status twd_sweep_tile_weights(const uint8_t *packed, int64_t N, int64_t K,
                                             uint8_t *tiled) {
    using twd::set_error;
    if (N < 0 || K < 0 || K % 64 != 0)
        return set_error(TWD_ERR_INVALID_ARG,
                         "sweep_tile_weights: need N >= 0 and K a non-negative multiple of 64");
    if ((N > 0 && K > 0) && (!packed || !tiled))
        return set_error(TWD_ERR_INVALID_ARG, "sweep_tile_weights: null pointer");
    const int64_t RB = K / 4;
    const int64_t tiles = (N + 15) / 16;
    const int64_t slices = (K + 255) / 256;
    for (int64_t t = 0; t < tiles; ++t)
        for (int64_t u = 0; u < slices; ++u)
            for (int l = 0; l < 64; ++l) {
                const int r = l & 15, g = l >> 4;
                const int64_t row = 16 * t + r;
                const int64_t col = 64 * u + 16 * g;
                uint8_t *dst = tiled + ((t * slices + u) * 64 + l) * 16;
                if (row < N && col < RB)
                    std::memcpy(dst, packed + row * RB + col, 16);
                else
                    std::memset(dst, 0, 16);
            }
    return TWD_OK;
}
