// Exercises the host side of libtwd -- the weight format (ternarize, pack,
// unpack, sweep tiling), the sweep planner and every entry point's argument
// checks -- for the AddressSanitizer / UndefinedBehaviorSanitizer build, with
// the device launches replaced by host_stubs.cpp.  Test infrastructure only.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "twd.h"

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main() {
    const int64_t N = 37, K = 320;
    std::vector<float> W(N * K);
    uint32_t r = 7;
    for (auto &w : W) {
        r = r * 1664525u + 1013904223u;
        w = (static_cast<float>(r >> 8) / 16777216.0f - 0.5f) * 0.04f;
    }
    std::vector<int8_t> codes(N * K), back(N * K);
    float gamma = 0.0f;
    CHECK(twd_ternarize_absmean(W.data(), N, K, codes.data(), &gamma) == TWD_OK);
    CHECK(twd_ternarize_absmean(W.data(), 0, K, codes.data(), &gamma) == TWD_OK);
    CHECK(twd_ternarize_absmean(W.data(), N, K, codes.data(), &gamma) == TWD_OK);
    std::vector<uint8_t> packed(N * K / 4);
    CHECK(twd_pack_ternary(codes.data(), N, K, packed.data()) == TWD_OK);
    CHECK(twd_unpack_ternary(packed.data(), N, K, back.data()) == TWD_OK);
    CHECK(std::memcmp(codes.data(), back.data(), codes.size()) == 0);
    packed[3] = 0xFF;
    CHECK(twd_unpack_ternary(packed.data(), N, K, back.data()) == TWD_ERR_BAD_CODE);
    codes[5] = 2;
    CHECK(twd_pack_ternary(codes.data(), N, K, packed.data()) == TWD_ERR_BAD_CODE);
    CHECK(twd_pack_ternary(codes.data(), N, 100, packed.data()) == TWD_ERR_INVALID_ARG);
    W[9] = NAN;
    CHECK(twd_ternarize_absmean(W.data(), N, K, codes.data(), &gamma) == TWD_ERR_INVALID_ARG);

    // sweep tiling
    const int64_t tb = twd_sweep_tiled_bytes(N, K);
    CHECK(tb == ((N + 15) / 16) * ((K + 255) / 256) * 1024);
    std::vector<uint8_t> tiled(tb);
    CHECK(twd_sweep_tile_weights(packed.data(), N, K, tiled.data()) == TWD_OK);
    CHECK(twd_sweep_tiled_bytes(N, 100) == -1);
    CHECK(twd_sweep_tile_weights(packed.data(), N, 100, tiled.data()) == TWD_ERR_INVALID_ARG);

    // sweep planner: a list with ragged shapes, an empty projection, 1..4
    // segments, and every width
    std::vector<twd_sweep_proj> projs(9);
    for (size_t i = 0; i < projs.size(); ++i) {
        twd_sweep_proj &p = projs[i];
        std::memset(&p, 0, sizeof p);
        const uintptr_t base = (uintptr_t(1) << 40) + (uintptr_t(i) << 26);
        p.wpacked = reinterpret_cast<const uint8_t *>(base);
        p.x_bf16 = reinterpret_cast<const uint16_t *>(base + (1 << 24));
        p.y = reinterpret_cast<float *>(base + (2 << 24));
        p.acc = (i % 2) ? reinterpret_cast<int32_t *>(base + (3 << 24)) : nullptr;
        p.K = 64 * (1 + (i * 37) % 128);
        p.nseg = 1 + i % 4;
        for (int s = 0; s < p.nseg; ++s) {
            p.seg_rows[s] = (i == 4) ? 0 : 1 + (i * 131 + s * 17) % 900;
            p.seg_gamma[s] = 0.01f * (s + 1);
        }
    }
    for (int64_t m = 1; m <= TWD_MAX_M; ++m) {
        int64_t bytes = 0;
        CHECK(twd_sweep_table_bytes(projs.data(), int(projs.size()), m, &bytes) == TWD_OK);
        std::vector<uint8_t> img(bytes);
        twd_sweep_plan plan;
        const void *dev = reinterpret_cast<const void *>(uintptr_t(1) << 44);
        CHECK(twd_sweep_encode(projs.data(), int(projs.size()), m, dev, img.data(), bytes,
                               &plan) == TWD_OK);
        CHECK(plan.nwg >= 1 && plan.table_bytes == bytes);
        CHECK(twd_sweep_encode(projs.data(), int(projs.size()), m, dev, img.data(), bytes - 1,
                               &plan) == TWD_ERR_INVALID_ARG);
        CHECK(twd_ternary_sweep(&plan, nullptr) == TWD_ERR_HIP);  // the stub launch fails
    }
    int64_t bytes = 0;
    CHECK(twd_sweep_table_bytes(projs.data(), int(projs.size()), 0, &bytes) ==
          TWD_ERR_UNSUPPORTED);
    CHECK(twd_sweep_table_bytes(nullptr, 3, 1, &bytes) == TWD_ERR_INVALID_ARG);
    projs[2].K = 100;
    CHECK(twd_sweep_table_bytes(projs.data(), int(projs.size()), 1, &bytes) ==
          TWD_ERR_UNSUPPORTED);
    CHECK(twd_ternary_sweep(nullptr, nullptr) == TWD_ERR_INVALID_ARG);

    // argument checks of the device entry points (nothing reaches a launch
    // but the calls the stubs refuse)
    const uint8_t *w = reinterpret_cast<const uint8_t *>(uintptr_t(1) << 36);
    const int8_t *xq = reinterpret_cast<const int8_t *>(uintptr_t(1) << 37);
    const float *xs = reinterpret_cast<const float *>(uintptr_t(1) << 38);
    float *y = reinterpret_cast<float *>(uintptr_t(1) << 39);
    CHECK(twd_ternary_linear(w, 1.0f, xq, xs, 17, 256, 64, nullptr, y, nullptr) ==
          TWD_ERR_UNSUPPORTED);
    CHECK(twd_ternary_linear(w, 1.0f, xq, xs, 4, 100, 64, nullptr, y, nullptr) ==
          TWD_ERR_UNSUPPORTED);
    CHECK(twd_ternary_linear(w + 1, 1.0f, xq, xs, 4, 256, 64, nullptr, y, nullptr) ==
          TWD_ERR_INVALID_ARG);
    CHECK(twd_ternary_linear(w, 1.0f, xq, xs, 4, 256, 64, nullptr, nullptr, nullptr) ==
          TWD_ERR_INVALID_ARG);
    CHECK(twd_ternary_linear(w, 1.0f, xq, xs, 0, 256, 64, nullptr, y, nullptr) == TWD_OK);
    CHECK(twd_ternary_linear(w, 1.0f, xq, xs, 4, 256, 64, nullptr, y, nullptr) == TWD_ERR_HIP);
    const int64_t rows[2] = {32, -1};
    const float gam[2] = {1.0f, 1.0f};
    CHECK(twd_ternary_linear_fused(w, 2, rows, gam, xq, xs, 4, 256, nullptr, y, nullptr) ==
          TWD_ERR_INVALID_ARG);
    CHECK(twd_ternary_linear_fused(w, 5, rows, gam, xq, xs, 4, 256, nullptr, y, nullptr) ==
          TWD_ERR_INVALID_ARG);
    CHECK(twd_ternary_linear_bf16(w, 1, rows, gam, reinterpret_cast<const uint16_t *>(xq), 5,
                                  256, nullptr, y, TWD_KERNEL_DOT, nullptr) ==
          TWD_ERR_UNSUPPORTED);
    const uint16_t *xb = reinterpret_cast<const uint16_t *>(xq);
    void *wsp = const_cast<float *>(xs);
    CHECK(twd_linear_bf16_workspace_bytes(16, 6912) == 16 * 6912 + 64);
    CHECK(twd_ternary_linear_bf16_ws(w, 1, rows, gam, xb, 16, 6912, nullptr, y, 0, wsp, 64,
                                     nullptr) == TWD_ERR_INVALID_ARG);
    CHECK(twd_ternary_linear_bf16_noalloc(w, 1, rows, gam, xb, 17, 256, nullptr, y, 0,
                                          nullptr) == TWD_ERR_UNSUPPORTED);
    CHECK(twd_ternary_linear_bf16_noalloc(w, 1, rows, gam, xb, 16, 6912, nullptr, y, 0,
                                          nullptr) == TWD_ERR_HIP);  // the stub lookup fails
    CHECK(twd_ternary_linear_bf16_noalloc(w, 1, rows, gam, xb, 4, 256, nullptr, y, 0,
                                          nullptr) == TWD_ERR_HIP);  // the stub launch fails
    CHECK(twd_select_kernel(1, 2560, 3840, 1) >= 1 && twd_select_kernel(0, 2560, 3840, 1) == -1);
    CHECK(twd_quantize_act(reinterpret_cast<const uint16_t *>(xq), 2, 12, const_cast<int8_t *>(xq),
                           const_cast<float *>(xs), nullptr) == TWD_ERR_UNSUPPORTED);
    CHECK(twd_projection_fp8(w, xs, reinterpret_cast<const uint16_t *>(xq), 17, 256, 8, y,
                             nullptr, nullptr, nullptr) == TWD_ERR_UNSUPPORTED);
    CHECK(twd_projection_bf16(reinterpret_cast<const uint16_t *>(w),
                              reinterpret_cast<const uint16_t *>(xq), 2, 100, 8, y,
                              nullptr) == TWD_ERR_UNSUPPORTED);
    CHECK(twd_stream_read(w, 17, reinterpret_cast<uint32_t *>(y), nullptr) ==
          TWD_ERR_INVALID_ARG);
    CHECK(twd_stream_copy(w, y, -16, nullptr) == TWD_ERR_INVALID_ARG);
    void *segs[2] = {const_cast<uint8_t *>(w), nullptr};
    const int32_t *cnt = reinterpret_cast<const int32_t *>(xs);
    CHECK(twd_kv_commit(segs, 2, 8, 2, 64, w, 4, cnt, cnt + 1, cnt + 4,
                        const_cast<int32_t *>(cnt) + 8, nullptr) == TWD_ERR_INVALID_ARG);
    CHECK(std::strlen(twd_last_error()) > 0);
    std::puts("host driver: ok");
    return 0;
}
