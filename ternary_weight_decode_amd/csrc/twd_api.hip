// C-ABI entry points: argument checks, the width dispatch, launches.
// Nothing here allocates, synchronizes or reads device memory, so every
// device call can be recorded into a HIP graph.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "twd_internal.h"

namespace twd {

namespace {
thread_local char g_error[512] = "";

bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

twd_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess)
        return TWD_OK;
    return set_error(TWD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxN = int64_t(1) << 30;

// Shared checks of the linear entry points; fills segs and N.  xscale is
// only required for the pre-quantized form (fused == false).
twd_status check_linear(const uint8_t *wpacked, int nseg,
                        const int64_t *seg_rows, const float *seg_gamma,
                        const void *act, bool fused, const float *xscale,
                        int64_t M, int64_t K, const int32_t *acc,
                        const float *y, int kernel, Segments *segs,
                        int64_t *N_out) {
    if (kernel != TWD_KERNEL_AUTO && kernel != TWD_KERNEL_DOT &&
        kernel != TWD_KERNEL_MFMA && kernel != TWD_KERNEL_MFMA_STAGED &&
        kernel != TWD_KERNEL_MFMA_TILE)
        return set_error(TWD_ERR_INVALID_ARG, "linear: unknown kernel %d", kernel);
    if (nseg < 1 || nseg > TWD_MAX_SEGMENTS)
        return set_error(TWD_ERR_INVALID_ARG, "linear: nseg=%d outside 1..%d",
                         nseg, TWD_MAX_SEGMENTS);
    if (!seg_rows || !seg_gamma)
        return set_error(TWD_ERR_INVALID_ARG, "linear: null segment table");
    int64_t N = 0;
    segs->nseg = nseg;
    for (int s = 0; s < TWD_MAX_SEGMENTS; ++s) {
        segs->bound[s] = 0;
        segs->gamma[s] = 0.0f;
    }
    for (int s = 0; s < nseg; ++s) {
        if (seg_rows[s] < 0)
            return set_error(TWD_ERR_INVALID_ARG, "linear: seg_rows[%d] < 0", s);
        N += seg_rows[s];
        if (N > kMaxN)
            return set_error(TWD_ERR_UNSUPPORTED, "linear: N > 2^30");
        segs->bound[s] = static_cast<int>(N);
        segs->gamma[s] = seg_gamma[s];
    }
    *N_out = N;
    if (M < 0 || M > TWD_MAX_M)
        return set_error(TWD_ERR_UNSUPPORTED, "linear: M=%lld outside 0..%d",
                         (long long)M, TWD_MAX_M);
    if (K < 64 || K > TWD_MAX_K || K % 64 != 0)
        return set_error(TWD_ERR_UNSUPPORTED,
                         "linear: K=%lld must be a multiple of 64 in 64..%d",
                         (long long)K, TWD_MAX_K);
    if (kernel == TWD_KERNEL_DOT && M > 4)
        return set_error(TWD_ERR_UNSUPPORTED, "linear: the dot kernel takes M <= 4");
    if (M == 0 || N == 0)
        return TWD_OK;
    if (!wpacked || !act || (!fused && !xscale))
        return set_error(TWD_ERR_INVALID_ARG, "linear: null input pointer");
    if (!acc && !y)
        return set_error(TWD_ERR_INVALID_ARG, "linear: acc and y are both NULL");
    if (!aligned(wpacked, 16) || !aligned(act, 16))
        return set_error(TWD_ERR_INVALID_ARG,
                         "linear: wpacked and the activations must be 16-byte aligned");
    if ((!fused && !aligned(xscale, 4)) || (acc && !aligned(acc, 4)) ||
        (y && !aligned(y, 4)))
        return set_error(TWD_ERR_INVALID_ARG,
                         "linear: xscale, acc and y must be 4-byte aligned");
    return TWD_OK;
}

}  // namespace

twd_status set_error(twd_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return st;
}

}  // namespace twd

using namespace twd;

extern "C" const char *twd_version(void) { return "twd 0.1.0 (gfx950)"; }

extern "C" const char *twd_last_error(void) { return g_error; }

extern "C" twd_status twd_quantize_act(const uint16_t *x_bf16, int64_t M,
                                       int64_t K, int8_t *xq, float *xscale,
                                       void *stream) {
    if (M < 0)
        return set_error(TWD_ERR_INVALID_ARG, "quantize_act: M < 0");
    if (K < 8 || K > 65536 || K % 8 != 0)
        return set_error(TWD_ERR_UNSUPPORTED,
                         "quantize_act: K=%lld must be a multiple of 8 in 8..65536",
                         (long long)K);
    if (M > 65535)
        return set_error(TWD_ERR_UNSUPPORTED, "quantize_act: M > 65535");
    if (M == 0)
        return TWD_OK;
    if (!x_bf16 || !xq || !xscale)
        return set_error(TWD_ERR_INVALID_ARG, "quantize_act: null pointer");
    if (!aligned(x_bf16, 16) || !aligned(xq, 16) || !aligned(xscale, 4))
        return set_error(TWD_ERR_INVALID_ARG,
                         "quantize_act: x and xq must be 16-byte aligned");
    return hip_status(launch_quantize_act(x_bf16, static_cast<int>(M),
                                          static_cast<int>(K), xq, xscale,
                                          as_stream(stream)),
                      "quantize_act launch");
}

namespace {

twd_status run_linear(const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
                      const float *seg_gamma, const void *act, bool fused,
                      const float *xscale, int64_t M, int64_t K, int32_t *acc,
                      float *y, int kernel, void *stream) {
    Segments segs;
    int64_t N = 0;
    twd_status st = check_linear(wpacked, nseg, seg_rows, seg_gamma, act, fused,
                                 xscale, M, K, acc, y, kernel, &segs, &N);
    if (st != TWD_OK || M == 0 || N == 0)
        return st;
    const LinearPlan plan = plan_linear(static_cast<int>(M), static_cast<int>(K),
                                        static_cast<int>(N), fused, kernel);
    return hip_status(launch_linear(plan, wpacked, act, fused, xscale,
                                    static_cast<int>(M), static_cast<int>(K),
                                    static_cast<int>(N), segs, acc, y,
                                    as_stream(stream)),
                      "linear launch");
}

}  // namespace

extern "C" twd_status twd_ternary_linear_fused_kernel(
    const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
    const float *seg_gamma, const int8_t *xq, const float *xscale, int64_t M,
    int64_t K, int32_t *acc, float *y, int kernel, void *stream) {
    return run_linear(wpacked, nseg, seg_rows, seg_gamma, xq, false, xscale, M,
                      K, acc, y, kernel, stream);
}

extern "C" twd_status twd_ternary_linear_bf16(
    const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
    const float *seg_gamma, const uint16_t *x_bf16, int64_t M, int64_t K,
    int32_t *acc, float *y, int kernel, void *stream) {
    return run_linear(wpacked, nseg, seg_rows, seg_gamma, x_bf16, true, nullptr,
                      M, K, acc, y, kernel, stream);
}

namespace {

// Where every workgroup of the fused launch would quantize a wide M x K
// block, the stand-alone quantizer followed by the pre-quantized linear is
// faster: from M = 14 on every 2B-class shape, and from M = 7 where
// K >= 4096 (the down projection, K = 6912: 6.8 against 7.6 us at M = 7,
// 8.3 against 10.6 us at M = 16, per launch, graph-replayed; at M = 6 one
// launch is still ahead, 6.2 against 6.6 us).
bool two_launch_pays(int64_t M, int64_t K) { return M >= 14 || (K >= 4096 && M >= 7); }

// Workspace of the two-launch form: the int8 rows [M][K], then (16-byte
// aligned) the fp32 scales [M].
int64_t quantized_offset(int64_t M, int64_t K) { return (M * K + 15) / 16 * 16; }

}  // namespace

extern "C" int64_t twd_linear_bf16_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || M > TWD_MAX_M || K < 64 || K > TWD_MAX_K || K % 64 != 0)
        return -1;
    return quantized_offset(M, K) + 4 * M;
}

namespace {

// The body shared by the workspace and the allocation-free forms, after the
// checks: one launch, or the quantizer into the workspace and then the int8
// linear from it.
twd_status linear_bf16_forms(const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
                             const float *seg_gamma, const uint16_t *x_bf16, int64_t M,
                             int64_t K, int64_t N, const Segments &segs, int32_t *acc,
                             float *y, int kernel, void *workspace, void *stream) {
    if (M == 0 || N == 0)
        return TWD_OK;
    if (!workspace || kernel != TWD_KERNEL_AUTO || !two_launch_pays(M, K))
        return run_linear(wpacked, nseg, seg_rows, seg_gamma, x_bf16, true, nullptr, M, K,
                          acc, y, kernel, stream);
    int8_t *xq = static_cast<int8_t *>(workspace);
    float *xs = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                          quantized_offset(M, K));
    hipError_t e = launch_quantize_act(x_bf16, static_cast<int>(M), static_cast<int>(K), xq,
                                       xs, as_stream(stream));
    if (e != hipSuccess)
        return hip_status(e, "quantize_act launch");
    const LinearPlan plan = plan_linear(static_cast<int>(M), static_cast<int>(K),
                                        static_cast<int>(N), false, TWD_KERNEL_AUTO);
    return hip_status(launch_linear(plan, wpacked, xq, false, xs, static_cast<int>(M),
                                    static_cast<int>(K), static_cast<int>(N), segs, acc, y,
                                    as_stream(stream)),
                      "linear launch");
}

}  // namespace

extern "C" twd_status twd_ternary_linear_bf16_ws(
    const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
    const float *seg_gamma, const uint16_t *x_bf16, int64_t M, int64_t K,
    int32_t *acc, float *y, int kernel, void *workspace, int64_t workspace_bytes,
    void *stream) {
    Segments segs;
    int64_t N = 0;
    twd_status st = check_linear(wpacked, nseg, seg_rows, seg_gamma, x_bf16, true, nullptr,
                                 M, K, acc, y, kernel, &segs, &N);
    if (st != TWD_OK)
        return st;
    if (workspace) {
        if (!aligned(workspace, 16))
            return set_error(TWD_ERR_INVALID_ARG, "linear_bf16_ws: workspace not 16-byte aligned");
        if (workspace_bytes < twd_linear_bf16_workspace_bytes(M, K))
            return set_error(TWD_ERR_INVALID_ARG,
                             "linear_bf16_ws: workspace of %lld bytes, %lld needed",
                             (long long)workspace_bytes,
                             (long long)twd_linear_bf16_workspace_bytes(M, K));
    }
    return linear_bf16_forms(wpacked, nseg, seg_rows, seg_gamma, x_bf16, M, K, N, segs, acc, y,
                             kernel, workspace, stream);
}

extern "C" twd_status twd_ternary_linear_bf16_noalloc(
    const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
    const float *seg_gamma, const uint16_t *x_bf16, int64_t M, int64_t K,
    int32_t *acc, float *y, int kernel, void *stream) {
    Segments segs;
    int64_t N = 0;
    twd_status st = check_linear(wpacked, nseg, seg_rows, seg_gamma, x_bf16, true, nullptr,
                                 M, K, acc, y, kernel, &segs, &N);
    if (st != TWD_OK)
        return st;
    const int64_t need = twd_linear_bf16_workspace_bytes(M, K);
    if (need < 0 || need > kNoAllocScratchBytes)
        return set_error(TWD_ERR_UNSUPPORTED,
                         "linear_bf16_noalloc: M=%lld, K=%lld needs %lld scratch bytes, "
                         "more than the %lld held",
                         (long long)M, (long long)K, (long long)need,
                         (long long)kNoAllocScratchBytes);
    if (M == 0 || N == 0)
        return TWD_OK;
    // Every call looks the array up, whichever form it runs, so the first
    // call on a device (of any shape) sets it up there.
    void *ws = nullptr;
    st = noalloc_scratch(stream, &ws);
    if (st != TWD_OK)
        return st;
    return linear_bf16_forms(wpacked, nseg, seg_rows, seg_gamma, x_bf16, M, K, N, segs, acc, y,
                             kernel, ws, stream);
}

extern "C" twd_status twd_ternary_linear_fused(
    const uint8_t *wpacked, int nseg, const int64_t *seg_rows,
    const float *seg_gamma, const int8_t *xq, const float *xscale, int64_t M,
    int64_t K, int32_t *acc, float *y, void *stream) {
    return twd_ternary_linear_fused_kernel(wpacked, nseg, seg_rows, seg_gamma,
                                           xq, xscale, M, K, acc, y,
                                           TWD_KERNEL_AUTO, stream);
}

extern "C" twd_status twd_ternary_linear(const uint8_t *wpacked, float gamma,
                                         const int8_t *xq, const float *xscale,
                                         int64_t M, int64_t K, int64_t N,
                                         int32_t *acc, float *y, void *stream) {
    if (N < 0)
        return set_error(TWD_ERR_INVALID_ARG, "linear: N < 0");
    const int64_t rows[1] = {N};
    const float gam[1] = {gamma};
    return twd_ternary_linear_fused_kernel(wpacked, 1, rows, gam, xq, xscale, M,
                                           K, acc, y, TWD_KERNEL_AUTO, stream);
}

extern "C" int twd_select_kernel(int64_t M, int64_t K, int64_t N, int bf16_input) {
    if (M < 1 || M > TWD_MAX_M || K < 64 || K > TWD_MAX_K || K % 64 != 0 ||
        N < 1 || N > kMaxN)
        return -1;
    return plan_linear(static_cast<int>(M), static_cast<int>(K),
                       static_cast<int>(N), bf16_input != 0, TWD_KERNEL_AUTO)
        .kernel;
}

namespace {

// Shared checks of the two projection roles.
twd_status check_projection(bool fp8, const void *w, const float *wscale, const void *x,
                            int64_t M, int64_t K, int64_t N, const float *y,
                            const uint8_t *xq, const float *xscale) {
    const char *name = fp8 ? "projection_fp8" : "projection_bf16";
    if (M < 0 || M > TWD_MAX_M)
        return set_error(TWD_ERR_UNSUPPORTED, "%s: M=%lld outside 0..%d", name,
                         (long long)M, TWD_MAX_M);
    if (N < 0 || N > (int64_t(1) << 24))
        return set_error(N < 0 ? TWD_ERR_INVALID_ARG : TWD_ERR_UNSUPPORTED,
                         "%s: N=%lld outside 0..2^24", name, (long long)N);
    const int kq = fp8 ? 16 : 8;
    if (K < kq || K > TWD_MAX_K_PROJECTION || K % kq != 0)
        return set_error(TWD_ERR_UNSUPPORTED, "%s: K=%lld must be a multiple of %d in %d..%d",
                         name, (long long)K, kq, kq, TWD_MAX_K_PROJECTION);
    if (projection_lds_bytes(fp8, static_cast<int>(M), static_cast<int>(K)) > 160 * 1024)
        return set_error(TWD_ERR_UNSUPPORTED,
                         "%s: M=%lld tokens of K=%lld do not fit the 160 KiB of LDS", name,
                         (long long)M, (long long)K);
    if (M == 0 || N == 0)
        return TWD_OK;
    if (!w || !x || !y || (fp8 && !wscale))
        return set_error(TWD_ERR_INVALID_ARG, "%s: null pointer", name);
    if (!aligned(w, 16) || !aligned(x, 16) || (fp8 && !aligned(wscale, 16)))
        return set_error(TWD_ERR_INVALID_ARG,
                         "%s: weights, activations and weight scales must be 16-byte aligned",
                         name);
    if (!aligned(y, 4) || (xq && !aligned(xq, 8)) || (xscale && !aligned(xscale, 4)))
        return set_error(TWD_ERR_INVALID_ARG,
                         "%s: y and xscale must be 4-byte aligned, xq 8-byte aligned", name);
    return TWD_OK;
}

}  // namespace

extern "C" twd_status twd_projection_fp8(const uint8_t *wq, const float *wscale,
                                         const uint16_t *x_bf16, int64_t M, int64_t K,
                                         int64_t N, float *y, uint8_t *xq, float *xscale,
                                         void *stream) {
    twd_status st = check_projection(true, wq, wscale, x_bf16, M, K, N, y, xq, xscale);
    if (st != TWD_OK || M == 0 || N == 0)
        return st;
    return hip_status(launch_projection(true, wq, wscale, x_bf16, static_cast<int>(M),
                                        static_cast<int>(K), static_cast<int>(N), y, xq,
                                        xscale, as_stream(stream)),
                      "projection_fp8 launch");
}

extern "C" twd_status twd_projection_bf16(const uint16_t *w_bf16, const uint16_t *x_bf16,
                                          int64_t M, int64_t K, int64_t N, float *y,
                                          void *stream) {
    twd_status st = check_projection(false, w_bf16, nullptr, x_bf16, M, K, N, y, nullptr,
                                     nullptr);
    if (st != TWD_OK || M == 0 || N == 0)
        return st;
    return hip_status(launch_projection(false, reinterpret_cast<const uint8_t *>(w_bf16),
                                        nullptr, x_bf16, static_cast<int>(M),
                                        static_cast<int>(K), static_cast<int>(N), y, nullptr,
                                        nullptr, as_stream(stream)),
                      "projection_bf16 launch");
}

extern "C" twd_status twd_kv_commit(void *const *segments, int nseg, int64_t seg0_positions,
                                    int64_t layers, int64_t row_bytes, const void *block,
                                    int64_t W, const int32_t *n_mat, const int32_t *n_new,
                                    const int32_t *state_in, int32_t *state_out,
                                    void *stream) {
    if (nseg < 1 || nseg > TWD_KV_MAX_SEGMENTS)
        return set_error(TWD_ERR_UNSUPPORTED, "kv_commit: nseg=%d outside 1..%d", nseg,
                         TWD_KV_MAX_SEGMENTS);
    if (seg0_positions < 1 || layers < 1 || row_bytes < 16 || row_bytes > 65536 ||
        row_bytes % 16 != 0 || W < 1 || W > TWD_KV_MAX_WIDTH)
        return set_error(TWD_ERR_INVALID_ARG,
                         "kv_commit: need C0 >= 1, layers >= 1, row_bytes %% 16 == 0 in "
                         "16..65536, 1 <= W <= %d",
                         TWD_KV_MAX_WIDTH);
    const int64_t capacity = seg0_positions * ((int64_t(1) << nseg) - 1);
    if (seg0_positions >= (int64_t(1) << 31) || capacity >= (int64_t(1) << 31))
        return set_error(TWD_ERR_UNSUPPORTED, "kv_commit: capacity C0 (2^nseg - 1) >= 2^31");
    if (2 * layers > 65535)
        return set_error(TWD_ERR_UNSUPPORTED, "kv_commit: layers > 32767");
    if (!segments || !block || !n_mat || !n_new || !state_in || !state_out)
        return set_error(TWD_ERR_INVALID_ARG, "kv_commit: null pointer");
    KvSegments segs{};
    for (int s = 0; s < nseg; ++s) {
        if (!segments[s] || !aligned(segments[s], 16))
            return set_error(TWD_ERR_INVALID_ARG,
                             "kv_commit: segment %d is null or not 16-byte aligned", s);
        segs.ptr[s] = segments[s];
    }
    segs.capacity = capacity;
    if (!aligned(block, 16) || !aligned(n_mat, 4) || !aligned(n_new, 4) ||
        !aligned(state_in, 4) || !aligned(state_out, 4))
        return set_error(TWD_ERR_INVALID_ARG, "kv_commit: misaligned pointer");
    const uintptr_t a = reinterpret_cast<uintptr_t>(state_in);
    const uintptr_t b = reinterpret_cast<uintptr_t>(state_out);
    if ((a < b ? b - a : a - b) < 16)
        return set_error(TWD_ERR_INVALID_ARG, "kv_commit: state_in and state_out overlap");
    return hip_status(launch_kv_commit(segs, static_cast<int>(seg0_positions),
                                       static_cast<int>(layers), static_cast<int>(row_bytes),
                                       block, static_cast<int>(W), n_mat, n_new, state_in,
                                       state_out, as_stream(stream)),
                      "kv_commit launch");
}

extern "C" twd_status twd_stream_read(const void *buf, int64_t bytes,
                                      uint32_t *sink, void *stream) {
    if (bytes < 0 || bytes % 16 != 0)
        return set_error(TWD_ERR_INVALID_ARG,
                         "stream_read: bytes must be a non-negative multiple of 16");
    if (bytes == 0)
        return TWD_OK;
    if (!buf || !sink || !aligned(buf, 16))
        return set_error(TWD_ERR_INVALID_ARG, "stream_read: bad pointer");
    if (bytes / 16 / 1024 >= (int64_t(1) << 31))
        return set_error(TWD_ERR_UNSUPPORTED, "stream_read: too large");
    return hip_status(launch_stream_read(buf, bytes, sink, as_stream(stream)),
                      "stream_read launch");
}

extern "C" twd_status twd_stream_copy(const void *src, void *dst, int64_t bytes,
                                      void *stream) {
    if (bytes < 0 || bytes % 16 != 0)
        return set_error(TWD_ERR_INVALID_ARG,
                         "stream_copy: bytes must be a non-negative multiple of 16");
    if (bytes == 0)
        return TWD_OK;
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16))
        return set_error(TWD_ERR_INVALID_ARG, "stream_copy: bad pointer");
    if (bytes / 16 / 1024 >= (int64_t(1) << 31))
        return set_error(TWD_ERR_UNSUPPORTED, "stream_copy: too large");
    return hip_status(launch_stream_copy(src, dst, bytes, as_stream(stream)),
                      "stream_copy launch");
}

extern "C" twd_status twd_sweep_table_bytes(const twd_sweep_proj *projs, int nproj, int64_t M,
                                            int64_t *bytes) {
    if (!bytes)
        return set_error(TWD_ERR_INVALID_ARG, "sweep_table_bytes: null bytes");
    return sweep_plan(projs, nproj, M, nullptr, nullptr, 0, bytes, nullptr);
}

extern "C" twd_status twd_sweep_encode(const twd_sweep_proj *projs, int nproj, int64_t M,
                                       const void *table_dev, void *table_host,
                                       int64_t table_bytes, twd_sweep_plan *plan) {
    if (!table_host)
        return set_error(TWD_ERR_INVALID_ARG, "sweep_encode: null host table");
    return sweep_plan(projs, nproj, M, table_dev, table_host, table_bytes, nullptr, plan);
}

extern "C" twd_status twd_ternary_sweep(const twd_sweep_plan *plan, void *stream) {
    if (!plan || !plan->table || !aligned(plan->table, 16))
        return set_error(TWD_ERR_INVALID_ARG, "sweep: null plan or misaligned table");
    if (plan->M < 1 || plan->M > TWD_MAX_M || plan->nproj < 1 || plan->nproj > 65536 ||
        plan->nwg < 1 || plan->lds_bytes < kSweepLdsHeader || plan->lds_bytes > 160 * 1024 ||
        plan->table_bytes < kSweepHeaderBytes + int64_t(plan->nproj) * int64_t(sizeof(SweepProj)) +
                                int64_t(plan->nwg) * int64_t(sizeof(SweepWork)))
        return set_error(TWD_ERR_INVALID_ARG, "sweep: plan fields out of range");
    return hip_status(launch_sweep(*plan, as_stream(stream)), "sweep launch");
}
