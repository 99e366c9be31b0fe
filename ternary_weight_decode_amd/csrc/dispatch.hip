// Width dispatch -- M1's choice of "packed low-bit operators by replay width
// and input/output dimensions" (BitMTP page, ai.info AI summary,
// "Methodology in Plain English", paragraph 3): the straight-line kernels
// while each wave's activation slices fit in registers, the staged
// matrix-core kernel otherwise, and its 16-row tiles per workgroup from the
// output size.  Straight-line flavour by measurement on the 2B and 4B layer
// shapes: at M = 1 the VALU dot kernel and the matrix-core one stream the
// weights equally fast (the dot kernel needs no zero block or B layout); from
// M = 2 the matrix cores are faster, since the VALU work grows with M.
#include "twd_internal.h"

namespace twd {

LinearPlan plan_linear(int M, int K, int N, int forced_kernel) {
    LinearPlan p;
    p.tiles = 1;
    int k = forced_kernel;
    if (k == TWD_KERNEL_AUTO)
        k = (M == 1 && narrow_supported(TWD_KERNEL_DOT, M, K)) ? TWD_KERNEL_DOT
                                                               : TWD_KERNEL_MFMA;
    if (k == TWD_KERNEL_MFMA && !narrow_supported(TWD_KERNEL_MFMA, M, K))
        k = TWD_KERNEL_MFMA_STAGED;
    p.kernel = k;
    if (k == TWD_KERNEL_MFMA_STAGED && (N + 15) / 16 >= 512)
        p.tiles = 2;
    return p;
}

hipError_t launch_linear(const LinearPlan &plan, const uint8_t *w,
                         const void *act, bool fused, const float *xscale,
                         int M, int K, int N, const Segments &segs,
                         int32_t *acc, float *y, hipStream_t stream) {
    if (plan.kernel == TWD_KERNEL_MFMA_STAGED)
        return launch_staged(plan.tiles, w, act, fused, xscale, M, K, N, segs, acc, y,
                             stream);
    return launch_narrow(plan.kernel, w, act, fused, xscale, M, K, N, segs, acc, y,
                         stream);
}

}  // namespace twd
