// Multi-projection sweep: one persistent launch runs a planned list of
// ternary projections (W2A8, per-token absmax int8 quantization of bf16
// activations inside), gfx950.
//
// What it computes (BitMTP page, ai.info AI summary): per projection, the
// packed low-bit operator of M1 ("Methodology in Plain English", paragraph
// 3) on ternary BitNet b1.58 weights ("What This Paper Is About") and 8-bit
// activations ("Main Findings", first bullet): q = per-token absmax int8 of
// x, acc[m][n] = sum_k q[m][k] t[n][k] in int32, y = acc * s_m * gamma(n).
// The result equals the one-launch bf16 linear on each projection.
//
// Why one launch.  On this chip a dependent kernel boundary costs more than
// streaming a whole small projection (a 2B-class O projection is 1.6 MB, a
// fifth of a microsecond of HBM time), so the launches of a layer set cost
// more than its weights.  Here the 16-row tiles of every projection of the
// list form one sequence, cut by the host planner into workgroup ranges of
// about equal bytes; each workgroup stages (quantizes) the activations of the
// at most four projections its range touches, once, and its waves then
// stream their tiles with the next passes' weight loads always in flight,
// across tile and projection boundaries, with no barrier and no kernel
// boundary until the list ends.
//
// Work split.  One workgroup of 12 or 16 waves per compute unit; its waves
// take the tiles of each of its projections one at a time from an LDS
// counter, so they run out of work together (a fixed share per wave left the
// compute unit with fewer and fewer loads in flight as its faster waves
// finished).  A tile (16 weight rows, all of K) is read in passes of four
// 256-wide K slices.  The weights come in the sweep's tiled layout
// (twd_sweep_tile_weights): tile t is a contiguous run of ceil(K / 256)
// blocks of 1 KiB, block u holding, at lane l = 16 g + r, the 16 packed
// bytes of tile row r at K offset 256 u + 64 g -- so each pass is four
// whole-line loads of 1 KiB each, and each load is the matrix-core A operand
// as it stands.  A register ring holds the pass being
// computed and the next passes' loads.  Each slice is decoded into four byte
// planes (codes c = t + 1 scaled 1, 4, 16, 1), the A operands of four
// v_mfma_i32_16x16x64_i8 with their own accumulators; B is the staged int8
// activation block (token columns at or past M read a zero block).  After a
// tile's last pass, lane (token r, group g) holds rows 4g..4g+3 for token r:
// sum q t = sum q c - sum q, then the dequant epilogue.
//
// Outputs.  Stores issued inside the weight stream, 64 bytes for each of up
// to 16 token rows per tile, slow the stream far more than their bytes
// would suggest.  Where the workgroup's outputs fit in LDS beside its staged
// activations (the planner decides), the epilogue keeps them there -- as the
// fp32 y and int32 acc values, or, where only that fits, as 24-bit
// accumulators from which y is recomputed, for as many of each span's first
// tiles as fit -- and the workgroup writes each token row's run of
// consecutive outputs at the end; only the tiles past those store in the
// stream.
#include <type_traits>

#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

constexpr int kRawBufferFlags = 0x00020000;  // raw buffer, 32-bit format
constexpr uint32_t kOutOfRange = 0x80000000u;

// The table is read-only for the whole launch: reading it through the
// constant address space gives scalar loads, which wait on the scalar
// counter instead of the vector-memory counter that tracks the weight ring.
template <typename T>
using cptr = const __attribute__((address_space(4))) T *;

// Field-wise copies out of the constant address space.
__device__ __forceinline__ SweepSpan span_at(cptr<SweepWork> wk, int s) {
    SweepSpan sp;
    sp.q = wk->span[s].q;
    sp.t0 = wk->span[s].t0;
    sp.t1 = wk->span[s].t1;
    sp.xoff = wk->span[s].xoff;
    sp.yoff = wk->span[s].yoff;
    sp.aoff = wk->span[s].aoff;
    sp.nd = wk->span[s].nd;
    return sp;
}

__device__ __forceinline__ Segments segs_of(cptr<SweepProj> P) {
    Segments sg;
    sg.nseg = P->segs.nseg;
#pragma unroll
    for (int i = 0; i < TWD_MAX_SEGMENTS; ++i) {
        sg.bound[i] = P->segs.bound[i];
        sg.gamma[i] = P->segs.gamma[i];
    }
    return sg;
}

// Staged activation layout: word 16 g + 4 d + j of a 64-word slice is stored
// at 16 g + 4 j + d, so one 16-byte read gives the B operand of plane j.
__device__ __forceinline__ int permuted_word(int w) {
    return (w & ~63) | (w & 48) | ((w & 3) << 2) | ((w >> 2) & 3);
}

// A pass: tile t of the span's projection, 256-wide slices kSweepLP p ..
// kSweepLP p + kSweepLP - 1.  The wave walks its tiles t0 + wave, t0 + wave
// + NW, ... and each tile's passes in order; two counters (tile, pass) stand
// for the pass index, so no division is needed.
struct PassPos {
    int t;
    int p;
};

template <int NW>
__device__ __forceinline__ void step(PassPos &c, int passes) {
    if (++c.p == passes) {
        c.p = 0;
        c.t += NW;
    }
}

// Weights of a span's projection, as the loads need them.
struct SpanW {
    const uint8_t *w;  // tiled weights
    int tile_bytes;    // 1 KiB per 256-wide slice
    int t1;            // end tile of the span
};

// Issue one pass's weight loads (kSweepLP slices of 1 KiB) into ring slot a;
// slices past K, and a pass past the span's last tile (an empty descriptor),
// load zeros without memory traffic, which keeps the count of loads in
// flight fixed.
__device__ __forceinline__ void issue(const SpanW &sw, const PassPos &c, int lane,
                                      uint4 (&a)[kSweepLP]) {
    const bool valid = c.t < sw.t1;
    const uint8_t *base = sw.w + static_cast<int64_t>(valid ? c.t : 0) * sw.tile_bytes;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(base), 0, valid ? sw.tile_bytes : 0, kRawBufferFlags);
#pragma unroll
    for (int i = 0; i < kSweepLP; ++i) {
        const uint32_t off = static_cast<uint32_t>(1024 * (kSweepLP * c.p + i) + 16 * lane);
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kWeightPolicy);
        a[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// Multiply one pass.  Every slice is multiplied, also those past K (their
// weights were loaded as zeros and their B operand is the zero block):
// consuming every ring register on every path keeps the compiler's
// vector-memory waits exact, so two passes stay in flight.
__device__ __forceinline__ void compute(int p, int slices, const uint8_t *bsrc, int ustep,
                                        const uint8_t *zero,
                                        const uint4 (&a)[kSweepLP], v4i &c0, v4i &c3,
                                        v4i &c4, v4i &c16) {
    if (p == 0) {
        c0 = v4i{0, 0, 0, 0};
        c3 = c0;
        c4 = c0;
        c16 = c0;
    }
#pragma unroll
    for (int i = 0; i < kSweepLP; ++i) {
        const int u = kSweepLP * p + i;
        const uint8_t *bu = u < slices ? bsrc + u * ustep : zero;
        const v4i b0 = *reinterpret_cast<const v4i *>(bu);
        const v4i b1 = *reinterpret_cast<const v4i *>(bu + 16);
        const v4i b2 = *reinterpret_cast<const v4i *>(bu + 32);
        const v4i b3 = *reinterpret_cast<const v4i *>(bu + 48);
        const v4i w = {static_cast<int>(a[i].x), static_cast<int>(a[i].y),
                       static_cast<int>(a[i].z), static_cast<int>(a[i].w)};
        const v4i p0 = w & static_cast<int>(kPlane0);
        const v4i p1 = w & static_cast<int>(kPlane1);
        const v4i p2 = w & static_cast<int>(kPlane2);
        const v4i p3 = (w >> 6) & static_cast<int>(kPlane0);
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p0, b0, c0, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p1, b1, c4, 0, 0, 0);
        c16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p2, b2, c16, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p3, b3, c3, 0, 0, 0);
    }
}

// Outputs of a span's projection, and this lane's token terms.
struct SpanOut {
    int32_t *acc;
    float *y;
    Segments segs;
    int N;
    int qs;     // row sum of q for token r
    float sc;   // scale of token r
    bool vec;   // 16-byte stores: N % 4 == 0 and both outputs 16-byte aligned
    int def;    // outputs gathered in LDS: 1 as fp32 y / int32 acc rows (ydef /
                // adef: [M][rows], null if absent), 2 as 24-bit accumulators
                // of the span's first nd tiles (ydef: [M][rows] of 3 bytes,
                // the later tiles stored in the stream); 0 stored in the stream
    uint8_t *ydef;
    uint8_t *adef;
    int t0, rows;  // the span's first tile and 16 x its deferred tile count
    int nd;
};

typedef float v4f __attribute__((ext_vector_type(4)));

// After a tile's last pass: lane (token r, group g) holds rows 4g .. 4g+3,
// four consecutive outputs of token r, written with one 16-byte store each
// for acc and y where the row layout allows it -- into the span's LDS rows
// when the workgroup defers its outputs, as values or as four 24-bit
// accumulators in three words (rows past N are never written out).
template <int M>
__device__ __forceinline__ void epilogue(const SpanOut &so, int t, int r, int g, const v4i &c0,
                                         const v4i &c3, const v4i &c4, const v4i &c16) {
    const v4i cc = c0 + c3 + (c4 >> 2) + (c16 >> 4);
    const int n0 = 16 * t + 4 * g;
    v4i tot;
    v4f yv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tot[i] = cc[i] - so.qs;
        yv[i] = static_cast<float>(tot[i]) * so.sc * row_gamma(so.segs, n0 + i);
    }
    if (r < M && n0 < so.N && so.def == 1) {
        const int e = 4 * (r * so.rows + 16 * (t - so.t0) + 4 * g);
        if (so.adef)
            *reinterpret_cast<v4i *>(so.adef + e) = tot;
        if (so.ydef)
            *reinterpret_cast<v4f *>(so.ydef + e) = yv;
    } else if (r < M && n0 < so.N && so.def == 2 && t - so.t0 < so.nd) {
        // |acc| <= 127 K < 2^23: the low 24 bits keep it
        uint32_t *d = reinterpret_cast<uint32_t *>(
            so.ydef + 3 * (r * so.rows + 16 * (t - so.t0) + 4 * g));
        const uint32_t u0 = static_cast<uint32_t>(tot[0]) & 0xFFFFFFu;
        const uint32_t u1 = static_cast<uint32_t>(tot[1]) & 0xFFFFFFu;
        const uint32_t u2 = static_cast<uint32_t>(tot[2]) & 0xFFFFFFu;
        const uint32_t u3 = static_cast<uint32_t>(tot[3]) & 0xFFFFFFu;
        d[0] = u0 | (u1 << 24);
        d[1] = (u1 >> 8) | (u2 << 16);
        d[2] = (u2 >> 16) | (u3 << 8);
    } else if (r < M && n0 < so.N) {
        const int64_t o = static_cast<int64_t>(r) * so.N + n0;
        if (so.vec) {
            // N % 4 == 0, so n0 < N means all four rows are in range
            if (so.acc)
                *reinterpret_cast<v4i *>(so.acc + o) = tot;
            if (so.y)
                *reinterpret_cast<v4f *>(so.y + o) = yv;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n0 + i < so.N) {
                    if (so.acc)
                        so.acc[o + i] = tot[i];
                    if (so.y)
                        so.y[o + i] = yv[i];
                }
        }
    }
}

// Write a deferred span's LDS rows ([M][rows], rows = 16 (t1 - t0), from
// output row 16 t0) to acc and y: 16-byte stores where N % 4 == 0 and both
// outputs are 16-byte aligned, else 4-byte stores; rows at or past N stay in
// LDS.
template <int M>
__device__ __forceinline__ void write_deferred(const uint8_t *smem, const SweepSpan &sp,
                                               cptr<SweepProj> P, int tid, int nthreads) {
    if (sp.yoff < 0 && sp.aoff < 0)
        return;
    const int N = P->N;
    const int rows = 16 * (sp.t1 - sp.t0);
    const int n0 = 16 * sp.t0;
    const int valid = N - n0 < rows ? N - n0 : rows;
    int32_t *acc = P->acc;
    float *y = P->y;
    const bool vec = (N & 3) == 0 &&
                     ((reinterpret_cast<uintptr_t>(acc) | reinterpret_cast<uintptr_t>(y)) & 15) ==
                         0;
    for (int r = 0; r < M; ++r) {
        const int64_t o = static_cast<int64_t>(r) * N + n0;
        const int e = 4 * r * rows;
        if (vec) {
            for (int j = 4 * tid; j < valid; j += 4 * nthreads) {
                if (sp.aoff >= 0)
                    *reinterpret_cast<v4i *>(acc + o + j) =
                        *reinterpret_cast<const v4i *>(smem + sp.aoff + e + 4 * j);
                if (sp.yoff >= 0)
                    *reinterpret_cast<v4f *>(y + o + j) =
                        *reinterpret_cast<const v4f *>(smem + sp.yoff + e + 4 * j);
            }
        } else {
            for (int j = tid; j < valid; j += nthreads) {
                if (sp.aoff >= 0)
                    acc[o + j] = *reinterpret_cast<const int32_t *>(smem + sp.aoff + e + 4 * j);
                if (sp.yoff >= 0)
                    y[o + j] = *reinterpret_cast<const float *>(smem + sp.yoff + e + 4 * j);
            }
        }
    }
}

// Write a packed deferred span's LDS rows ([M][rows] 24-bit accumulators, rows =
// 16 nd, from output row 16 t0) to acc and y, y recomputed from the
// accumulator with the epilogue's own fp32 operations (so the same bits):
// each thread takes four consecutive outputs of a token row, 16-byte stores
// where N % 4 == 0 and both outputs are 16-byte aligned, else 4-byte stores;
// rows at or past N stay in LDS.  scale: the span's per-token scales.
static_assert(127 * TWD_MAX_K < (1 << 23), "a deferred accumulator fits in 24 bits");

template <int M>
__device__ __forceinline__ void write_packed(const uint8_t *smem, const SweepSpan &sp,
                                             cptr<SweepProj> P, const float *scale, int tid,
                                             int nthreads) {
    if (sp.yoff < 0 || sp.nd <= 0)
        return;
    const int N = P->N;
    const int rows = 16 * sp.nd;
    const int n0 = 16 * sp.t0;
    const int valid = N - n0 < rows ? N - n0 : rows;
    int32_t *acc = P->acc;
    float *y = P->y;
    const Segments segs = segs_of(P);
    const bool vec = (N & 3) == 0 &&
                     ((reinterpret_cast<uintptr_t>(acc) | reinterpret_cast<uintptr_t>(y)) & 15) ==
                         0;
    for (int r = 0; r < M; ++r) {
        const int64_t o = static_cast<int64_t>(r) * N + n0;
        const float sc = scale[r];
        for (int j = 4 * tid; j < valid; j += 4 * nthreads) {
            const uint32_t *d =
                reinterpret_cast<const uint32_t *>(smem + sp.yoff + 3 * (r * rows + j));
            const uint32_t w0 = d[0], w1 = d[1], w2 = d[2];
            v4i a;
            a[0] = static_cast<int32_t>(w0 << 8) >> 8;
            a[1] = static_cast<int32_t>(((w0 >> 24) | (w1 << 8)) << 8) >> 8;
            a[2] = static_cast<int32_t>(((w1 >> 16) | (w2 << 16)) << 8) >> 8;
            a[3] = static_cast<int32_t>(w2) >> 8;
            v4f yv;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                yv[i] = static_cast<float>(a[i]) * sc * row_gamma(segs, n0 + j + i);
            if (vec) {
                if (acc)
                    *reinterpret_cast<v4i *>(acc + o + j) = a;
                if (y)
                    *reinterpret_cast<v4f *>(y + o + j) = yv;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (j + i < valid) {
                        if (acc)
                            acc[o + j + i] = a[i];
                        if (y)
                            y[o + j + i] = yv[i];
                    }
            }
        }
    }
}

// The next tile of span s from the workgroup's LDS counter: one lane takes
// it, the whole wave gets it as a uniform value.
__device__ __forceinline__ int fetch_tile(int *ctr, int s, int lane) {
    int t = 0;
    if (lane == 0)
        t = __hip_atomic_fetch_add(&ctr[s], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(t);
}

// The issue side's position: span s, tile t, pass p.  A wave takes the tiles
// of span s one at a time from the span's counter; when the span runs out it
// moves on to the next span.  Past the last span the position holds an empty
// descriptor (loads return zeros without memory traffic) and s = nspan.
struct DynCursor {
    SpanW w;
    int t, p, passes, s;

    __device__ __forceinline__ void begin(int s0, int nspan, cptr<SweepWork> wk,
                                          cptr<SweepProj> projs, int *ctr, int lane) {
        for (s = s0; s < nspan; ++s) {
            const SweepSpan sp = span_at(wk, s);
            t = fetch_tile(ctr, s, lane);
            if (t < sp.t1) {
                const cptr<SweepProj> P = projs + sp.q;
                w.w = P->w;
                w.tile_bytes = 1024 * P->slices;
                w.t1 = sp.t1;
                passes = P->passes;
                p = 0;
                return;
            }
        }
        w.w = nullptr;
        w.tile_bytes = 0;
        w.t1 = 0;
        t = 0;
        p = 0;
        passes = 1;
    }

    __device__ __forceinline__ void advance(int nspan, cptr<SweepWork> wk, cptr<SweepProj> projs,
                                            int *ctr, int lane) {
        if (s >= nspan)
            return;
        if (++p < passes)
            return;
        p = 0;
        t = fetch_tile(ctr, s, lane);
        if (t < w.t1)
            return;
        begin(s + 1, nspan, wk, projs, ctr, lane);
    }
};

// Built for SW resident waves per SIMD (512 / SW registers per lane) with a
// register ring of kS passes.
template <int M, int NW, int kS, int SW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(SW)))
void sweep_kernel(const SweepHeader *header_g, const SweepProj *projs_g,
                  const SweepWork *work_g, uint32_t check) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *zero = smem;  // 64 zero bytes
    uint32_t *st_max = reinterpret_cast<uint32_t *>(smem + 64);  // [span][16]
    int32_t *st_sum = reinterpret_cast<int32_t *>(st_max + kSweepMaxSpans * 16);
    float *st_scale = reinterpret_cast<float *>(st_sum + kSweepMaxSpans * 16);
    uint8_t *xbase = smem + kSweepLdsHeader;

    const cptr<SweepHeader> header = (cptr<SweepHeader>)header_g;
    const cptr<SweepProj> projs = (cptr<SweepProj>)projs_g;
    if (header->check != check)
        return;  // the table does not belong to this plan: write nothing

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const cptr<SweepWork> wk = (cptr<SweepWork>)work_g + blockIdx.x;
    const int nspan = wk->nspan;

    // The issue side f runs kS - 1 passes ahead of the compute side, from
    // span to span, so the ring never drains at a span boundary; each ring
    // slot carries the span, tile and pass it holds.  The first kS - 1
    // passes go out before the staging at M <= 12 (after the first span's
    // activation loads), so the first weights arrive while the activations
    // are quantized; above, in 128 registers, the staging holds too many (a
    // wave per token row, 16 rounds of loads) for the ring to be live across
    // it.  The counters hold each span's next tile.
    constexpr bool kEarly = M <= 12;
    int *ctr = reinterpret_cast<int *>(st_scale + kSweepMaxSpans * 16);
    DynCursor f;
    uint4 ring[kS][kSweepLP];
    int tag_s[kS], tag_t[kS], tag_p[kS];
    auto prologue = [&]() {
        f.begin(0, nspan, wk, projs, ctr, lane);
#pragma unroll
        for (int k = 0; k < kS - 1; ++k) {
            issue(f.w, PassPos{f.t, f.p}, lane, ring[k]);
            tag_s[k] = f.s;
            tag_t[k] = f.t;
            tag_p[k] = f.p;
            f.advance(nspan, wk, projs, ctr, lane);
        }
    };

    // 1. stage the activations of every span.  Token row m is quantized by
    //    kWpr waves (a whole wave per row once M >= NW; waves past the last
    //    row idle): their lanes take the row's chunks of 8 activations in
    //    turn, all loaded in one round trip and kept in registers from the
    //    absmax to the rounding.  With one wave per row the absmax and the row
    //    sum are wave reductions and need no barrier.
    constexpr int kWpr = M >= NW ? 1 : NW / M;
    constexpr int kLanes = 64 * kWpr;
    // chunk rounds per lane: K <= 8192
    constexpr int kRounds = (TWD_MAX_K / 8 + kLanes - 1) / kLanes;
    const int m = wave / kWpr;               // this wave's token row
    const int cl = 64 * (wave % kWpr) + lane;  // its first chunk of the row
    if (tid < 16 + 2 * kSweepMaxSpans * 16)
        reinterpret_cast<uint32_t *>(smem)[tid] = 0u;
    if (tid < kSweepMaxSpans) {
        int t0 = 0;
#pragma unroll
        for (int k = 0; k < kSweepMaxSpans; ++k)
            if (k == tid && k < nspan)
                t0 = wk->span[k].t0;
        ctr[tid] = t0;
    }
    __syncthreads();
    auto stage = [&](int s, auto early) {
        const SweepSpan sp = span_at(wk, s);
        const cptr<SweepProj> P = projs + sp.q;
        const int K = P->K;
        const int C = K >> 3;
        // Every round is loaded and every load feeds the absmax, on every
        // path: rounds past the row end, and waves without a row (an empty
        // descriptor), load zeros without memory traffic.  Loads or uses
        // behind a branch would leave the compiler unsure which loads are
        // still in flight at the next span, and it would then wait for all of
        // them before each new load.
        const bool has_row = m < M;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(P->x) + (has_row ? static_cast<int64_t>(m) * K : 0), 0,
            has_row ? K * 2 : 0, kRawBufferFlags);
        uint4 v[kRounds];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            const int ch = cl + kLanes * i;
            const uint32_t off = ch < C ? static_cast<uint32_t>(16 * ch) : kOutOfRange;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            v[i] = make_uint4(x[0], x[1], x[2], x[3]);
        }
        if constexpr (decltype(early)::value)
            prologue();
        u16x2 am = {0, 0};
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            am = absmax_pair(am, v[i].x);
            am = absmax_pair(am, v[i].y);
            am = absmax_pair(am, v[i].z);
            am = absmax_pair(am, v[i].w);
        }
        uint32_t amax = wave_umax(absmax_bits(am));
        // the rounding skips rounds that hold no chunk below C (uniformly
        // over the wave)
        const int first = cl - lane;
        if constexpr (kWpr > 1) {
            if (m < M && lane == 0)
                __hip_atomic_fetch_max(&st_max[s * 16 + m], amax, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            __syncthreads();  // absmax of every token row of this span
            if (m < M)
                amax = st_max[s * 16 + m];
        }
        if (m < M) {
            const float a_m = __uint_as_float(amax);
            // correctly rounded fp32 divisions (build flag), as in the
            // stand-alone quantizer; an all-zero row quantizes to zeros
            const float inv = a_m > 0.0f ? 127.0f / a_m : 0.0f;
            if (cl == 0)
                st_scale[s * 16 + m] = a_m / 127.0f;
            uint8_t *row = xbase + sp.xoff + m * P->stride;
            int sq = 0;
#pragma unroll
            for (int i = 0; i < kRounds; ++i) {
                if (first + kLanes * i < C) {
                    const int ch = cl + kLanes * i;
                    const uint32_t q0 = quant4(v[i].x, v[i].y, inv);
                    const uint32_t q1 = quant4(v[i].z, v[i].w, inv);
                    if (ch < C) {
                        *reinterpret_cast<uint32_t *>(row + 4 * permuted_word(2 * ch)) = q0;
                        *reinterpret_cast<uint32_t *>(row + 4 * permuted_word(2 * ch + 1)) = q1;
                    }
                    sq = sdot4(q0, kOnes, sq);
                    sq = sdot4(q1, kOnes, sq);
                }
            }
            sq = wave_sum(sq);
            if (lane == 0) {
                if constexpr (kWpr == 1)
                    st_sum[s * 16 + m] = sq;
                else
                    __hip_atomic_fetch_add(&st_sum[s * 16 + m], sq, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    };
    if (nspan > 0)
        stage(0, std::integral_constant<bool, kEarly>{});
    else if constexpr (kEarly)
        prologue();  // the same loads on both paths (all past the end here)
    for (int s = 1; s < nspan; ++s)
        stage(s, std::false_type{});
    __syncthreads();  // staged rows, row sums and scales

    // 2. stream: the waves of the workgroup take the tiles of each span from
    //    its LDS counter, one tile at a time, span after span, so they all run
    //    out of work within about a tile of each other.  Each ring slot
    //    carries the span, tile and pass it holds; the compute side reads
    //    them back.  The loads run kS - 1 passes ahead, across spans.
    int cs = 0;  // span whose outputs the compute side holds
    SpanOut so;
    const uint8_t *bsrc = zero;
    int ustep = 0, slices = 1, cpasses = 1;
    auto load_span = [&](int s) {
        const SweepSpan sp = span_at(wk, s);
        const cptr<SweepProj> P = projs + sp.q;
        slices = P->slices;
        cpasses = P->passes;
        so.acc = P->acc;
        so.y = P->y;
        so.segs = segs_of(P);
        so.N = P->N;
        so.qs = st_sum[s * 16 + r];
        so.sc = st_scale[s * 16 + r];
        so.vec = (so.N & 3) == 0 &&
                 ((reinterpret_cast<uintptr_t>(so.acc) | reinterpret_cast<uintptr_t>(so.y)) &
                  15) == 0;
        bsrc = r < M ? xbase + sp.xoff + r * P->stride + 64 * g : zero;
        ustep = r < M ? 256 : 0;
        so.def = wk->defer;
        so.ydef = sp.yoff >= 0 ? smem + sp.yoff : nullptr;
        so.adef = sp.aoff >= 0 ? smem + sp.aoff : nullptr;
        so.t0 = sp.t0;
        so.nd = sp.nd;
        so.rows = 16 * (so.def == 2 ? sp.nd : sp.t1 - sp.t0);
    };
    load_span(0);  // (with no span: the table's zeroed entry, never used)
    v4i c0 = {0, 0, 0, 0}, c3 = c0, c4 = c0, c16 = c0;
#define TWD_SWEEP_ISSUE(SLOT)                                                  \
    issue(f.w, PassPos{f.t, f.p}, lane, ring[SLOT]);                           \
    tag_s[SLOT] = f.s;                                                         \
    tag_t[SLOT] = f.t;                                                         \
    tag_p[SLOT] = f.p;                                                         \
    f.advance(nspan, wk, projs, ctr, lane);
#define TWD_SWEEP_STEP(CUR)                                                    \
    TWD_SWEEP_ISSUE(((CUR) + kS - 1) % kS)                                     \
    if (tag_s[CUR] != cs && tag_s[CUR] < nspan) {                              \
        cs = tag_s[CUR];                                                       \
        load_span(cs);                                                         \
    }                                                                          \
    compute(tag_p[CUR], slices, bsrc, ustep, zero, ring[CUR], c0, c3, c4, c16); \
    if (tag_s[CUR] < nspan && tag_p[CUR] == cpasses - 1)                       \
        epilogue<M>(so, tag_t[CUR], r, g, c0, c3, c4, c16);
    if constexpr (!kEarly)
        prologue();
    for (;;) {
#pragma unroll
        for (int k = 0; k < kS; ++k) {
            TWD_SWEEP_STEP(k)
        }
        bool pending = f.s < nspan;
#pragma unroll
        for (int k = 0; k < kS - 1; ++k)
            pending = pending || tag_s[k] < nspan;
        if (!pending)
            break;
    }
#undef TWD_SWEEP_STEP
#undef TWD_SWEEP_ISSUE

    // 3. deferred outputs: once every wave is done, each token row's run of
    //    each span goes out in one pass over consecutive addresses.
    if (wk->defer) {
        __syncthreads();
        for (int s = 0; s < nspan; ++s)
            if (wk->defer == 2)
                write_packed<M>(smem, span_at(wk, s), projs + wk->span[s].q, st_scale + s * 16,
                                tid, 64 * NW);
            else
                write_deferred<M>(smem, span_at(wk, s), projs + wk->span[s].q, tid, 64 * NW);
    }
}

using Fn = void (*)(const SweepHeader *, const SweepProj *, const SweepWork *, uint32_t);

template <int... Ms>
Fn pick(int M) {
    Fn fn = nullptr;
    ((M == Ms ? (void)(fn = &sweep_kernel<Ms, sweep_waves(Ms), sweep_ring(Ms),
                                          sweep_simd_waves(Ms)>)
              : (void)0),
     ...);
    return fn;
}

}  // namespace

hipError_t launch_sweep(const twd_sweep_plan &plan, hipStream_t stream) {
    Fn fn = pick<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(plan.M);
    if (!fn)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), plan.lds_bytes);
    if (e != hipSuccess)
        return e;
    const uint8_t *t = static_cast<const uint8_t *>(plan.table);
    const SweepHeader *h = reinterpret_cast<const SweepHeader *>(t);
    const SweepProj *p = reinterpret_cast<const SweepProj *>(t + kSweepHeaderBytes);
    const SweepWork *w = reinterpret_cast<const SweepWork *>(
        t + kSweepHeaderBytes + static_cast<int64_t>(plan.nproj) * sizeof(SweepProj));
    hipLaunchKernelGGL(fn, dim3(plan.nwg), dim3(64 * sweep_waves(plan.M)), plan.lds_bytes, stream, h, p,
                       w, plan.check);
    return hipGetLastError();
}

}  // namespace twd
