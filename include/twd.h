/*
 * twd.h -- C ABI of the MI355X (gfx950) W2A8 ternary linear library.
 *
 * The library computes the packed W2A8 linear layer that BitMTP's
 * width-specialized low-bit execution runs at the narrow token widths that
 * block-parallel multi-token prediction produces (page "BitMTP: When
 * Multi-Token Prediction Meets Low-Bit Large Language Models", ai.info AI
 * summary): M = 1 for autoregressive steps, M = 2..16 for drafted-block
 * verification ("Methodology in Plain English", paragraphs 2-3: the verifier
 * runs the anchor plus the whole draft through the model; M1 picks packed
 * low-bit operators by replay width and input/output dimensions).  Weights
 * are ternary (BitNet b1.58, "What This Paper Is About"); the setting is W2A8:
 * 2-bit weights, 8-bit activations ("Main Findings", first bullet).
 *
 * Conventions for every call:
 *   - W is [N][K] (output rows x input columns), x is [M][K], y = x W^T.
 *   - The caller owns every buffer; the library keeps no pointer after a call
 *     returns and allocates nothing.  Device calls are asynchronous on
 *     `stream` (a hipStream_t; NULL means the null stream): buffers must stay
 *     alive until that stream's work completes.  Device calls neither
 *     synchronize nor read device memory on the host, so they may be
 *     captured into a HIP graph.
 *   - Arguments are checked before anything is launched.  On a non-OK status
 *     nothing was launched (or, for TWD_ERR_HIP, the launch failed) and
 *     twd_last_error() returns a message for the calling thread.
 *   - Integer results are deterministic: two calls on the same inputs give
 *     the same bits.
 */
#ifndef TWD_H
#define TWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TWD_OK = 0,
    TWD_ERR_INVALID_ARG = 1, /* null pointer, negative size, misaligned buffer */
    TWD_ERR_UNSUPPORTED = 2, /* shape outside what the kernels handle */
    TWD_ERR_BAD_CODE = 3,    /* weight code outside {-1, 0, +1} or field == 3 */
    TWD_ERR_HIP = 4          /* the HIP runtime reported an error */
} twd_status;

/* Limits of the device kernels. */
#define TWD_MAX_M 16          /* token rows per call */
#define TWD_MAX_K 8192        /* input width (activation rows are staged in LDS) */
#define TWD_MAX_SEGMENTS 4    /* independently scaled row segments (fused) */
#define TWD_MAX_K_PROJECTION 4096 /* input width of the fast / critical projections */
#define TWD_KV_MAX_SEGMENTS 24    /* KV segments of the accepted-prefix commit */
#define TWD_KV_MAX_WIDTH 64       /* block rows one KV commit can take */

/* Kernel families of the linear; TWD_KERNEL_AUTO lets the width dispatch
 * choose (M1's "select by replay width and input/output dimensions"). */
typedef enum {
    TWD_KERNEL_AUTO = 0,
    /* row-owner VALU kernel: 2-bit decode in registers + v_dot4 int8;
     * M <= 4 */
    TWD_KERNEL_DOT = 1,
    /* straight-line matrix-core kernel (v_mfma_i32_16x16x64_i8): 16 rows
     * per workgroup, K split over 4, 8 or 16 waves by M and K */
    TWD_KERNEL_MFMA = 2,
    /* matrix cores with separate activation-staging waves: any M, K */
    TWD_KERNEL_MFMA_STAGED = 3,
    /* matrix cores, one 16-row tile per wave over all of K and 64 rows per
     * workgroup (activations staged once per 64 rows); K <= 3072, else the
     * staged kernel */
    TWD_KERNEL_MFMA_TILE = 4
} twd_kernel;

/* Library version string; never NULL. */
const char *twd_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *twd_last_error(void);

/* ------------------------------------------------------------------------
 * Weight format (host, offline).
 *
 * Ternary code c = t + 1 (0, 1, 2; 3 is invalid), two bits per weight.  Row
 * n occupies K/4 bytes; rows are contiguous.  Its K/16 little-endian 32-bit
 * words each hold sixteen weights k = 16 i + e with e = 4 j + b (j, b in
 * 0..3): the code of element e sits at bit 8 b + 2 j.  So masking a word
 * with 0x03030303 << 2j yields four byte lanes holding the codes of
 * elements 4j .. 4j+3, which line up with one 32-bit word of int8
 * activations.  The pages call the execution "packed W2A8" ("Methodology in
 * Plain English", last paragraph) but give no layout; this one is chosen
 * for byte-wise dot products and matrix-core operands.
 * ---------------------------------------------------------------------- */

/* Absmean ternarization of one tensor W[N][K] (fp32, host memory):
 * gamma = mean |W| (summed in double in row-major order, rounded once to
 * fp32), codes = clamp(rint(W / gamma), -1, 1) with an fp32 division and
 * ties to even; gamma == 0 gives all-zero codes.  BitNet b1.58's rule; the
 * pages name the model but not the formula.  codes: host int8 [N][K].
 * Errors: INVALID_ARG for null pointers, negative sizes or a non-finite W. */
twd_status twd_ternarize_absmean(const float *W, int64_t N, int64_t K,
                                 int8_t *codes, float *gamma);

/* Pack host codes int8 [N][K] in {-1, 0, +1} into host bytes [N][K/4].
 * Errors: INVALID_ARG (null, N < 0, K < 0, K % 16 != 0), BAD_CODE. */
twd_status twd_pack_ternary(const int8_t *codes, int64_t N, int64_t K,
                            uint8_t *packed);

/* Inverse of twd_pack_ternary.  Errors: INVALID_ARG, BAD_CODE on a field
 * holding the invalid code 3. */
twd_status twd_unpack_ternary(const uint8_t *packed, int64_t N, int64_t K,
                              int8_t *codes);

/* ------------------------------------------------------------------------
 * Device calls.
 * ---------------------------------------------------------------------- */

/* Per-token absmax int8 quantization ("Main Findings": 8-bit activations).
 * x_bf16: device bf16 bit patterns [M][K]; xq: device int8 [M][K];
 * xscale: device fp32 [M].  For each row: a = max |x|, inv = 127 / a (fp32,
 * correctly rounded), xq = clamp(rint(x * inv), -127, 127), xscale = a / 127;
 * a == 0 gives xq = 0 and xscale = 0.  Non-finite x is outside the contract.
 * Shapes: 0 <= M <= 65535 (M == 0 is a no-op), 8 <= K <= 65536, K % 8 == 0.
 * Alignment: x_bf16 and xq 16-byte aligned. */
twd_status twd_quantize_act(const uint16_t *x_bf16, int64_t M, int64_t K,
                            int8_t *xq, float *xscale, void *stream);

/* W2A8 ternary linear: acc[m][n] = sum_k xq[m][k] * t[n][k] in int32
 * (exact), y[m][n] = acc[m][n] * xscale[m] * gamma in fp32.  The packed
 * low-bit operator that M1 selects by replay width and input/output
 * dimensions (page "BitMTP: When Multi-Token Prediction Meets Low-Bit Large
 * Language Models", ai.info AI summary, "Methodology in Plain English", last
 * paragraph), in the W2A8 setting ("Main Findings", first bullet): ternary
 * weights with one absmean scale, int8 activations with one scale per token
 * (BitNet b1.58, named in "What This Paper Is About").  The pages give no
 * rounding order for the dequantization; the two fp32 products are taken in
 * the order written.
 * wpacked: device packed weights [N][K/4] (format above); xq, xscale: the
 * outputs of twd_quantize_act; acc (int32 [M][N]) and y (fp32 [M][N]) are
 * device outputs, either may be NULL (not both).
 * Shapes: 0 <= M <= 16 (M == 0 is a no-op), N >= 0 (N == 0 is a no-op),
 * 64 <= K <= TWD_MAX_K with K % 64 == 0.  Alignment: wpacked and xq 16 bytes,
 * acc and y 4 bytes.  The kernel is chosen by (M, K, N). */
twd_status twd_ternary_linear(const uint8_t *wpacked, float gamma,
                              const int8_t *xq, const float *xscale,
                              int64_t M, int64_t K, int64_t N,
                              int32_t *acc, float *y, void *stream);

/* Fused projections (Q/K/V, gate/up): one launch over the concatenated
 * output rows.  The operator of twd_ternary_linear (same page and passages)
 * applied to projections that read the same activations; each keeps its own
 * absmean scale, as BitNet b1.58 ternarizes each weight tensor on its own.
 * The pages do not describe the fusion; it is a launch-count choice of this
 * library and changes no result.  seg_rows / seg_gamma are HOST arrays of nseg (1..4) entries:
 * segment s covers the next seg_rows[s] rows and is dequantized with
 * seg_gamma[s].  They are copied into the kernel arguments, so a captured
 * graph keeps them.  N = sum of seg_rows; other arguments as above. */
twd_status twd_ternary_linear_fused(const uint8_t *wpacked, int nseg,
                                    const int64_t *seg_rows,
                                    const float *seg_gamma,
                                    const int8_t *xq, const float *xscale,
                                    int64_t M, int64_t K,
                                    int32_t *acc, float *y, void *stream);

/* As twd_ternary_linear_fused with the kernel family forced (tests and
 * measurement of the width crossover).  kernel = TWD_KERNEL_AUTO behaves
 * exactly like twd_ternary_linear_fused. */
twd_status twd_ternary_linear_fused_kernel(const uint8_t *wpacked, int nseg,
                                           const int64_t *seg_rows,
                                           const float *seg_gamma,
                                           const int8_t *xq,
                                           const float *xscale, int64_t M,
                                           int64_t K, int32_t *acc, float *y,
                                           int kernel, void *stream);

/* One launch for a whole projection: the per-token absmax int8
 * quantization of bf16 activations x_bf16 (device [M][K], 16-byte aligned),
 * with exactly the arithmetic of twd_quantize_act, fused into the ternary
 * linear over nseg row segments.  acc / y and the segment tables as in
 * twd_ternary_linear_fused; kernel as in twd_ternary_linear_fused_kernel.
 * Reading of the pages: BitNet b1.58 quantizes activations inside every
 * ternary layer ("What This Paper Is About" names the backbone), so the
 * quantizer belongs to the layer's launch. */
twd_status twd_ternary_linear_bf16(const uint8_t *wpacked, int nseg,
                                   const int64_t *seg_rows,
                                   const float *seg_gamma,
                                   const uint16_t *x_bf16, int64_t M,
                                   int64_t K, int32_t *acc, float *y,
                                   int kernel, void *stream);

/* Bytes of the workspace twd_ternary_linear_bf16_ws uses for (M, K): the
 * int8 rows [M][K], then (at the next 16-byte boundary) the fp32 scales
 * [M].  -1 for M outside 0..TWD_MAX_M or K outside the linear's limits. */
int64_t twd_linear_bf16_workspace_bytes(int64_t M, int64_t K);

/* twd_ternary_linear_bf16 with the form picked by width and shape (M1 picks
 * the operator by replay width and by the layer's dimensions: BitMTP page,
 * "Methodology in Plain English", paragraph 3).  Where every workgroup of
 * the fused launch would quantize a wide M x K block -- M >= 14, or M >= 7
 * with K >= 4096 -- and kernel is TWD_KERNEL_AUTO, it runs two launches
 * instead: twd_quantize_act into the workspace, then the pre-quantized
 * linear (twd_ternary_linear_fused) from it.  Results are identical either
 * way (acc bit for bit, y the same fp32 evaluation).  workspace: device,
 * 16-byte aligned, at least twd_linear_bf16_workspace_bytes(M, K) bytes,
 * owned by the caller; calls that share a workspace must not overlap.
 * workspace = NULL always runs the one-launch form.  Other arguments and
 * errors as twd_ternary_linear_bf16, plus INVALID_ARG for a misaligned or
 * short workspace. */
twd_status twd_ternary_linear_bf16_ws(const uint8_t *wpacked, int nseg,
                                      const int64_t *seg_rows,
                                      const float *seg_gamma,
                                      const uint16_t *x_bf16, int64_t M,
                                      int64_t K, int32_t *acc, float *y,
                                      int kernel, void *workspace,
                                      int64_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * twd_ternary_linear_bf16_ws with the library's own workspace, a static
 * device array of 131136 bytes per device (the workspace of M = TWD_MAX_M,
 * K = TWD_MAX_K), held until the process ends.  Same arguments, results
 * and errors as twd_ternary_linear_bf16_ws with a workspace, plus
 * UNSUPPORTED where twd_linear_bf16_workspace_bytes(M, K) exceeds that
 * array, and INVALID_ARG if the stream belongs to a device other than the
 * current one.  The first call on a device with M, N > 0, whatever form it
 * runs, looks up the array's address there (hipGetSymbolAddress; no
 * allocation); make that first call outside graph capture.  Nothing is allocated, freed or
 * synchronized.  All calls on one device share its array: calls that
 * overlap on one device (different streams not ordered against each other,
 * or host threads launching at once) race on it and give wrong results;
 * order them on one stream.  Nothing needs clearing between calls (the
 * quantizer writes every byte the linear then reads). */
twd_status twd_ternary_linear_bf16_noalloc(const uint8_t *wpacked, int nseg,
                                           const int64_t *seg_rows,
                                           const float *seg_gamma,
                                           const uint16_t *x_bf16, int64_t M,
                                           int64_t K, int32_t *acc, float *y,
                                           int kernel, void *stream);

/* The kernel family the width dispatch picks for (M, K, N), without
 * launching anything: for twd_ternary_linear_bf16 if bf16_input != 0, else
 * for the int8 entry points (the choice can differ where the quantization
 * inside the launch changes which kernel is fastest).  Returns a twd_kernel
 * value other than TWD_KERNEL_AUTO, or -1 if the shape is unsupported. */
int twd_select_kernel(int64_t M, int64_t K, int64_t N, int bf16_input);

/* ------------------------------------------------------------------------
 * Role-dependent output projections.  The M1 paragraph of "Methodology in
 * Plain English" pairs cheaper "fast" projections for drafting with careful
 * "critical" ones for autoregressive steps and verification, and names FP8
 * draft projections (on H20).  The pages define neither; the readings here:
 * fast = OCP E4M3 weights with one fp32 scale per output row and E4M3
 * activations with one scale per token; critical = bf16 weights and
 * activations.  Both accumulate in fp32.  W is [N][K] row-major (output
 * rows x input columns), x is [M][K] bf16 bit patterns, y is fp32 [M][N].
 * ---------------------------------------------------------------------- */

/* Per-output-row FP8 quantization of weights W[N][K] (fp32, host memory):
 * a = max_k |W[n][k]|, inv = 448 / a (fp32 division), codes[n][k] =
 * E4M3(W[n][k] * inv) (fp32 multiply, round to nearest, ties to even),
 * scale[n] = a / 448 (fp32 division); a == 0 gives zero codes and scale 0.
 * codes: host uint8 [N][K]; scale: host fp32 [N].
 * Errors: INVALID_ARG for null pointers, negative sizes or a non-finite W. */
twd_status twd_quantize_fp8_rows(const float *W, int64_t N, int64_t K,
                                 uint8_t *codes, float *scale);

/* Fast projection: y[m][n] = (sum_k dec(xq[m][k]) dec(wq[n][k])) * xs[m] *
 * wscale[n] in fp32, where the per-token FP8 quantization of x_bf16 (xs =
 * max|x| / 448, xq = E4M3(x * (448 / max|x|)), as twd_quantize_fp8_rows
 * does per row) happens inside the launch.  wq: device E4M3 codes [N][K]
 * (16-byte aligned); wscale: device fp32 [N] (16-byte aligned); x_bf16:
 * device [M][K] (16-byte aligned); y: device fp32 [M][N].  xq (device uint8
 * [M][K], 8-byte aligned) and xscale (device fp32 [M]) may be NULL; if given
 * they receive the activation codes and scales.  Sums are accumulated in
 * fp32 (products of E4M3 values are exact), so y differs from the exact
 * value by at most the fp32 summation error.
 * Shapes: 0 <= M <= 16, 0 <= N <= 2^24 (either zero is a no-op), 16 <= K
 * <= TWD_MAX_K_PROJECTION with K % 16 == 0; else UNSUPPORTED. */
twd_status twd_projection_fp8(const uint8_t *wq, const float *wscale,
                              const uint16_t *x_bf16, int64_t M, int64_t K,
                              int64_t N, float *y, uint8_t *xq, float *xscale,
                              void *stream);

/* Critical projection: y[m][n] = sum_k x[m][k] w[n][k] over bf16 values,
 * fp32 accumulation.  w_bf16: device [N][K]; x_bf16: device [M][K] (both
 * 16-byte aligned); y: device fp32 [M][N].  Shapes as twd_projection_fp8
 * but 8 <= K with K % 8 == 0. */
twd_status twd_projection_bf16(const uint16_t *w_bf16, const uint16_t *x_bf16,
                               int64_t M, int64_t K, int64_t N, float *y,
                               void *stream);

/* ------------------------------------------------------------------------
 * Accepted-prefix KV commit over shared, geometrically sized segments
 * ("Methodology in Plain English", paragraph 3: a state triple -- committed
 * prefix, materialized causal KV length, pending suffix -- kept consistent by
 * a length identity, and one physical KV buffer per segment, viewed by every
 * captured graph, with capacities growing geometrically; "Key
 * Contributions", item 1).  The pages write out neither the identity nor the
 * layout; the readings here:
 *
 * State: device int32[4] = {P committed tokens, L of them with stored causal
 * KV rows, S = P - L pending, error}.  Identity P == L + S, L >= 0, S >= 0.
 * Segments: segment s (0 <= s < nseg) holds C0 * 2^s positions, following
 * segments 0..s-1; its buffer is [layers][2 (K, V)][C0 * 2^s][row_bytes].
 * Block: the rows a pass computed for W consecutive positions starting at L,
 * [layers][2][W][row_bytes].
 * Commit: with n_mat and n_new read from device memory, rows 0 .. n_mat-1 of
 * the block are stored at positions L .. L+n_mat-1, and state_out = {P +
 * n_new, L + n_mat, P + n_new - L - n_mat, 0}.  A verification pass uses
 * n_mat = S + accepted drafts and n_new = accepted + 1 (the verifier's own
 * next token stays pending); an autoregressive step n_mat = n_new = 1; a
 * commit without KV (confidence-only) n_mat = 0.
 * Errors found on the device write nothing to the segments and set
 * state_out = state_in with error = 1 (identity broken on entry), 2 (n_mat
 * outside 0..W, n_new < 0, P + n_new >= 2^31 or L + n_mat > P + n_new) or 3
 * (L + n_mat beyond the segments); an error already set in state_in is
 * carried over.
 * ---------------------------------------------------------------------- */

/* segments: HOST array of nseg device pointers (16-byte aligned), copied into
 * the kernel arguments; seg0_positions = C0 >= 1; layers >= 1; row_bytes a
 * multiple of 16 in 16..65536; block: device, 16-byte aligned; 1 <= W <=
 * TWD_KV_MAX_WIDTH; n_mat, n_new: device int32; state_in, state_out: device
 * int32[4] that do not overlap (alternate two state words between calls).
 * Asynchronous on stream; reads no device memory on the host, so it can be
 * captured into a graph.  Errors: INVALID_ARG (null, misaligned, overlap,
 * bad sizes), UNSUPPORTED (nseg outside 1..TWD_KV_MAX_SEGMENTS, capacity
 * C0 * (2^nseg - 1) >= 2^31, 2 * layers > 65535). */
twd_status twd_kv_commit(void *const *segments, int nseg, int64_t seg0_positions,
                         int64_t layers, int64_t row_bytes, const void *block,
                         int64_t W, const int32_t *n_mat, const int32_t *n_new,
                         const int32_t *state_in, int32_t *state_out, void *stream);

/* ------------------------------------------------------------------------
 * Multi-projection sweep: one persistent launch over many independent
 * ternary projections (each the one-launch bf16 form above: per-token absmax
 * int8 quantization inside, W2A8 contraction, dequant epilogue).  M1 picks
 * packed low-bit operators by replay width ("Methodology in Plain English",
 * paragraph 3); a decode step's layer set at one width is a fixed list of
 * such operators, and graph replay needs fixed shapes and addresses (the same
 * paragraph), so the list is planned once and replayed.  Where the
 * projections of the list do not consume each other's outputs (the
 * synthetic layer sets, or independent projections of one layer), one launch
 * streams all their packed weights without a kernel boundary between them.
 * Results are those of twd_ternary_linear_bf16 on each projection: acc
 * bit-identical, y within the fp32 evaluation of acc * s_m * gamma.
 * ---------------------------------------------------------------------- */

/* Bytes of a projection's weights in the sweep's tiled layout: ceil(N / 16)
 * tiles of ceil(K / 256) KiB; -1 if N < 0 or K is not a non-negative
 * multiple of 64. */
int64_t twd_sweep_tiled_bytes(int64_t N, int64_t K);

/* Reorder packed weights [N][K/4] (the format above; host memory) into the
 * sweep's tiled layout (host memory, twd_sweep_tiled_bytes(N, K) bytes):
 * tile t (rows 16 t .. 16 t + 15) is a contiguous run of ceil(K / 256)
 * blocks of 1 KiB; block u holds, at position l = 16 g + r (16 bytes each),
 * packed bytes 64 u + 16 g .. 64 u + 16 g + 15 of row 16 t + r.  Zero bytes
 * pad rows past N and bytes past K / 4; a zero field contributes nothing to
 * the sweep's sums.  So every 1 KiB block is one whole-line load that is
 * the matrix-core operand as it stands.  Host, offline, like packing.
 * Errors: INVALID_ARG (null pointers, N < 0, K not a multiple of 64). */
twd_status twd_sweep_tile_weights(const uint8_t *packed, int64_t N, int64_t K,
                                  uint8_t *tiled);

/* One projection of a sweep.  wpacked: device, the projection's packed
 * weights in the sweep's tiled layout (twd_sweep_tile_weights; 16-byte
 * aligned);
 * x_bf16: device [M][K] bf16 bit patterns (16-byte aligned); acc: device
 * int32 [M][N] or NULL; y: device fp32 [M][N] or NULL (not both NULL; 4-byte
 * aligned); segments as in twd_ternary_linear_fused (N = sum of seg_rows,
 * which may be 0).  64 <= K <= TWD_MAX_K, K % 64 == 0.  Outputs of different
 * projections must not overlap each other or any input. */
typedef struct {
    const uint8_t *wpacked;
    const uint16_t *x_bf16;
    int32_t *acc;
    float *y;
    int64_t K;
    int64_t nseg;
    int64_t seg_rows[TWD_MAX_SEGMENTS];
    float seg_gamma[TWD_MAX_SEGMENTS];
} twd_sweep_proj;

/* A planned sweep (filled by twd_sweep_encode; the caller keeps it). */
typedef struct {
    const void *table;      /* device copy of the table image */
    int64_t table_bytes;
    int64_t weight_bytes;   /* sum of N K / 4 over the projections */
    int32_t nproj, M, nwg, lds_bytes;
    uint32_t check;         /* also stored in the table; the kernel compares */
    int32_t reserved[3];
} twd_sweep_plan;

/* Bytes of the table image for this list (host only, launches nothing).
 * Errors as twd_sweep_encode. */
twd_status twd_sweep_table_bytes(const twd_sweep_proj *projs, int nproj, int64_t M,
                                 int64_t *bytes);

/* Plan the sweep and write its table image into HOST memory table_host
 * (table_bytes from twd_sweep_table_bytes); the plan records table_dev, the
 * DEVICE buffer (16-byte aligned, table_bytes long, owned by the caller) into
 * which the caller copies the image before the first twd_ternary_sweep.  Host
 * only.  1 <= M <= TWD_MAX_M, 1 <= nproj <= 65536.
 * Errors: INVALID_ARG (null or misaligned pointers, bad segments, a table
 * that is too small), UNSUPPORTED (K or M outside the limits). */
twd_status twd_sweep_encode(const twd_sweep_proj *projs, int nproj, int64_t M,
                            const void *table_dev, void *table_host, int64_t table_bytes,
                            twd_sweep_plan *plan);

/* Run every projection of the plan in one launch, asynchronously on stream.
 * The device table, weights, activations and outputs must stay unchanged in
 * place (inputs) and alive until the stream's work completes.  The kernel
 * writes nothing if the device table does not carry the plan's check value.
 * Allocates nothing, reads no device memory on the host: capturable into a
 * HIP graph.  Errors: INVALID_ARG (null plan, bad plan fields), HIP. */
twd_status twd_ternary_sweep(const twd_sweep_plan *plan, void *stream);

/* Measurement helper: a plain streaming read of `bytes` device bytes
 * (16-byte aligned, bytes % 16 == 0) that stores nothing but a guard word
 * into sink (device, >= 1024 bytes).  Its launch duration is the
 * achievable-bandwidth reference for a kernel moving the same bytes. */
twd_status twd_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                           void *stream);

/* Measurement helper: a plain copy of `bytes` device bytes from src to dst
 * (both 16-byte aligned, not overlapping, bytes % 16 == 0).  It reads and
 * writes exactly `bytes` each, which calibrates hardware byte counters. */
twd_status twd_stream_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TWD_H */
