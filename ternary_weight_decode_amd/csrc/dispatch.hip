// Width dispatch -- M1's choice of "packed low-bit operators by replay width
// and input/output dimensions" (BitMTP page, ai.info AI summary,
// "Methodology in Plain English", paragraph 3): the VALU dot kernel for the
// narrowest widths, the matrix-core kernel for the wider verification
// widths, and the number of 16-row tiles per workgroup from the output size.
#include "twd_internal.h"

namespace twd {

LinearPlan plan_linear(int M, int K, int N, int forced_kernel) {
    (void)K;
    LinearPlan p;
    p.kernel = forced_kernel != TWD_KERNEL_AUTO
                   ? forced_kernel
                   : (M <= 4 ? TWD_KERNEL_DOT : TWD_KERNEL_MFMA);
    const int tiles = (N + 15) / 16;
    p.tiles = (p.kernel == TWD_KERNEL_MFMA && tiles >= 512) ? 2 : 1;
    return p;
}

hipError_t launch_linear(const LinearPlan &plan, const uint8_t *w,
                         const void *act, bool fused, const float *xscale,
                         int M, int K, int N, const Segments &segs,
                         int32_t *acc, float *y, hipStream_t stream) {
    if (plan.kernel == TWD_KERNEL_DOT)
        return launch_dot(plan.tiles, w, act, fused, xscale, M, K, N, segs, acc, y,
                          stream);
    return launch_mfma(plan.tiles, w, act, fused, xscale, M, K, N, segs, acc, y,
                       stream);
}

}  // namespace twd
