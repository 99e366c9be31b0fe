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
