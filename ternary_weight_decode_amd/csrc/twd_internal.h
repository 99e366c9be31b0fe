// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "twd.h"

namespace twd {

// Per-launch description of the fused row segments.  bound[s] is the first
// row after segment s (cumulative), gamma[s] its weight scale.  Passed by
// value as a kernel argument.
struct Segments {
    int nseg;
    int bound[TWD_MAX_SEGMENTS];
    float gamma[TWD_MAX_SEGMENTS];
};

// Launch parameters the width dispatch chose for one linear call.
struct LinearPlan {
    int kernel;  // TWD_KERNEL_DOT, _MFMA, _MFMA_TILE or _MFMA_STAGED
    int tiles;   // 16-row tiles per workgroup (staged kernel)
};

// The straight-line MFMA kernel holds each wave's activation slices in
// registers (M x U words, U = 256-wide K slices per wave): it exists for
// M * U <= 48, with 4, 8 or 16 waves sharing K.
constexpr bool narrow_fits(int M, int U) { return U >= 1 && U <= 8 && M * U <= 48; }

// Thread-local error message; returns `st` for convenient chaining.
twd_status set_error(twd_status st, const char *fmt, ...);

// The static workspace of twd_ternary_linear_bf16_noalloc: its size, and its
// address on the device that runs `stream` (which must be the current one),
// looked up once per device.  Sets the error text on failure.
constexpr int64_t kNoAllocScratchBytes = int64_t(TWD_MAX_M) * TWD_MAX_K + 4 * TWD_MAX_M;
twd_status noalloc_scratch(void *stream, void **out);

LinearPlan plan_linear(int M, int K, int N, bool bf16_input, int forced_kernel);

hipError_t launch_quantize_act(const uint16_t *x, int M, int K, int8_t *xq,
                               float *xscale, hipStream_t stream);

// act is int8 xq [M][K] with its scales xscale, or, when fused, bf16 x
// [M][K] quantized inside the kernel (xscale unused).
hipError_t launch_linear(const LinearPlan &plan, const uint8_t *w,
                         const void *act, bool fused, const float *xscale,
                         int M, int K, int N, const Segments &segs,
                         int32_t *acc, float *y, hipStream_t stream);

// Straight-line MFMA kernel (ternary_narrow.hip), for the (M, K)
// narrow_supported accepts; narrow_waves gives its waves per workgroup
// (waves = 0), or waves = 4, 8, 16 forces a count (the launch fails if the
// slices per wave then exceed the register budget).
int narrow_waves(int M, int K);
bool narrow_supported(int M, int K);
hipError_t launch_narrow(const uint8_t *w, const void *act, bool fused,
                         const float *xscale, int M, int K, int N,
                         const Segments &segs, int32_t *acc, float *y,
                         hipStream_t stream, int waves = 0);
// Row-owner VALU dot kernel (ternary_rows.hip): M <= 4, any K; the launch
// shape (rows per wave, waves per workgroup) comes from rows_shape.
void rows_shape(int M, int K, int N, int *rows_per_wave, int *waves);
hipError_t launch_rows(const uint8_t *w, const void *act, bool fused, const float *xscale,
                       int M, int K, int N, const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream);
// Tile-owner MFMA kernel (ternary_tile.hip): 64 rows per workgroup, one
// 16-row tile per wave over all of K; K <= 3072.
bool tile_supported(int M, int K);
hipError_t launch_tile(const uint8_t *w, const void *act, bool fused, const float *xscale,
                       int M, int K, int N, const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream);
// Staged matrix-core kernel (ternary_staged.hip): any M <= 16 and K.
hipError_t launch_staged(int tiles, const uint8_t *w, const void *act, bool fused,
                       const float *xscale, int M, int K, int N,
                       const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream);

// Role-dependent output projections (projection.hip): fp8 selects the fast
// role (E4M3 weight codes with per-row scales, activations quantized to
// E4M3 per token inside), else the critical role (bf16 weights).  K is
// padded to the kernel's chunk; the staged activations take
// projection_lds_bytes of LDS.  xq_out / xs_out (fast role, nullable)
// receive the activation codes and scales.
int projection_padded_k(bool fp8, int K);
int projection_lds_bytes(bool fp8, int M, int K);
hipError_t launch_projection(bool fp8, const uint8_t *w, const float *wscale,
                             const uint16_t *x, int M, int K, int N, float *y,
                             uint8_t *xq_out, float *xs_out, hipStream_t stream);

// Accepted-prefix KV commit (kv_commit.hip): the segment buffers as a kernel
// argument, and the total positions they hold.
struct KvSegments {
    void *ptr[TWD_KV_MAX_SEGMENTS];
    int64_t capacity;
};
hipError_t launch_kv_commit(const KvSegments &segs, int C0, int layers, int row_bytes,
                            const void *block, int W, const int32_t *n_mat,
                            const int32_t *n_new, const int32_t *state_in, int32_t *state_out,
                            hipStream_t stream);

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                              hipStream_t stream);
hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes,
                              hipStream_t stream);


// Multi-projection sweep (ternary_sweep.hip, planned by sweep_plan.cpp).  The
// device table is a header, one SweepProj per projection and one SweepWork per
// workgroup; its layout is private to the library.
constexpr int kSweepMaxSpans = 4;      // projections one workgroup stages
constexpr int kSweepLP = 4;            // 256-wide K slices per pass
// Per width: waves per workgroup, resident waves per SIMD the kernel is
// built for (its register budget: 512 / that many registers per lane), and
// the passes of its register ring (one computed, the rest in flight).  One
// workgroup fills a compute unit, so all the compute unit's waves share one
// tile counter: 12 waves (three per SIMD, up to 168 registers) while the
// staging has a wave for every token row, M <= 12; 16 waves (four per SIMD,
// 128 registers) above.  The planner aims for 4 x sweep_simd_waves(M) /
// sweep_waves(M) workgroups on each of kSweepCUs compute units.
constexpr int kSweepCUs = 256;
constexpr int sweep_waves(int m) { return m <= 12 ? 12 : 16; }
constexpr int sweep_simd_waves(int m) { return m <= 12 ? 3 : 4; }
constexpr int sweep_ring(int) { return 2; }
constexpr int kSweepHeaderBytes = 64;  // table header
constexpr uint32_t kSweepMagic = 0x53445754u;  // "TWDS"
// LDS: zero block (64 B), then per-span absmax, row-sum and scale words
// (kSweepMaxSpans x 16 each), the next-tile counter of each span (16 B),
// then the staged activation rows, then (where they fit) the deferred
// outputs: per span, [M][16 (t1 - t0)] values of y and of acc, or where
// those do not fit, [M][16 nd] accumulators of 24 bits (3 bytes each, four
// consecutive ones in three words) for the span's first nd tiles.
constexpr int kSweepLdsHeader = 64 + 3 * kSweepMaxSpans * 16 * 4 + 16;

struct SweepProj {       // 96 bytes
    const uint8_t *w;    // packed [N][K/4]
    const uint16_t *x;   // bf16 [M][K]
    int32_t *acc;        // [M][N] or null
    float *y;            // [M][N] or null
    int K;
    int N;
    int passes;          // passes per 16-row tile (kSweepLP slices each)
    int slices;          // 256-wide K slices, ceil(K / 256)
    int stride;          // LDS bytes per staged token row
    Segments segs;
    int pad[2];
};
static_assert(sizeof(SweepProj) == 96, "SweepProj layout");

struct SweepSpan {       // tiles [t0, t1) of projection q, activations at xoff
    int q, t0, t1, xoff;
    int yoff, aoff;      // LDS byte offsets of the deferred y / acc rows, or -1; with
                         // packed deferral yoff holds the 24-bit accumulators
    int nd;              // packed deferral: the span's first nd tiles are deferred
    int pad;
};

struct SweepWork {       // 144 bytes: one workgroup's spans, in order
    int nspan;
    int defer;           // the spans' outputs gathered in LDS, written at the end:
                         // 1 as fp32 y / int32 acc rows, 2 as 24-bit accumulators
                         // (of each span's first nd tiles; the rest stored in the stream)
    int pad[2];
    SweepSpan span[kSweepMaxSpans];
};
static_assert(sizeof(SweepWork) == 144, "SweepWork layout");

struct SweepHeader {     // 64 bytes
    uint32_t magic, check;
    int nproj, nwg, M, lds;
    int proj_off, work_off;
    int64_t weight_bytes;
    int pad[6];
};
static_assert(sizeof(SweepHeader) == kSweepHeaderBytes, "SweepHeader layout");

// Host planner: checks every projection, splits the tiles over workgroups and
// writes the table image.  table_host == nullptr only sizes the table.
twd_status sweep_plan(const twd_sweep_proj *projs, int nproj, int64_t M, const void *table_dev,
                      void *table_host, int64_t table_bytes, int64_t *bytes_needed,
                      twd_sweep_plan *plan);
hipError_t launch_sweep(const twd_sweep_plan &plan, hipStream_t stream);

}  // namespace twd
