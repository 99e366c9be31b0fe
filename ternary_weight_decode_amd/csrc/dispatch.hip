// Width dispatch -- M1's choice of "packed low-bit operators by replay width
// and input/output dimensions" (BitMTP page, ai.info AI summary,
// "Methodology in Plain English", paragraph 3).  By measurement on the 2B
// layer shapes: at M = 1 the row-owner VALU dot kernel is fastest (whole
// 128-byte lines per load, no cross-wave reduction), and at M = 2 still for
// int8 activations; from there the matrix cores win, since the VALU work
// grows with M.  A wide output (at least ~200 workgroups of 64 rows) takes
// the tile-owner kernel, which quantizes the activations once per 64 rows
// instead of once per 16 and loads whole 128-byte lines: from M = 2 with
// the quantization inside, from M = 3 for int8 activations (at M = 2 the dot
// kernel leads there).  Otherwise the straight-line MFMA kernel.  That kernel runs four waves per 16 rows while
// each wave's activation slices fit in registers; past that it splits K over
// 8 or 16 waves, which beats the staged kernel on int8 activations but not
// with the bf16 quantization inside (every one of the extra waves repeats
// its share of it), so a bf16 input there takes the staged kernel.  The dot
// kernel picks its own launch shape from N; the staged kernel takes two
// 16-row tiles per workgroup from 512 tiles up.
#include "twd_internal.h"

namespace twd {

LinearPlan plan_linear(int M, int K, int N, bool bf16_input, int forced_kernel) {
    LinearPlan p;
    p.tiles = 1;
    int k = forced_kernel;
    if (k == TWD_KERNEL_AUTO) {
        if (M == 1 || (M == 2 && !bf16_input))
            k = TWD_KERNEL_DOT;
        else if (M >= (bf16_input ? 2 : 3) && N / 64 >= 200 && tile_supported(M, K))
            k = TWD_KERNEL_MFMA_TILE;
        else if (bf16_input && narrow_waves(M, K) != 4)
            k = TWD_KERNEL_MFMA_STAGED;
        else
            k = TWD_KERNEL_MFMA;
    }
    if (k == TWD_KERNEL_MFMA && !narrow_supported(M, K))
        k = TWD_KERNEL_MFMA_STAGED;
    if (k == TWD_KERNEL_MFMA_TILE && !tile_supported(M, K))
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
    if (plan.kernel == TWD_KERNEL_MFMA_TILE)
        return launch_tile(w, act, fused, xscale, M, K, N, segs, acc, y, stream);
    if (plan.kernel == TWD_KERNEL_DOT)
        return launch_rows(w, act, fused, xscale, M, K, N, segs, acc, y, stream);
    return launch_narrow(w, act, fused, xscale, M, K, N, segs, acc, y, stream);
}

}  // namespace twd
