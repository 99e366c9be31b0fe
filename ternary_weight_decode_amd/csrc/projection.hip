// Role-dependent output projections, gfx950: the "fast" FP8 projection for
// drafting and the "critical" bf16 one for autoregressive steps and
// verification (BitMTP page, ai.info AI summary, "Methodology in Plain
// English", the paragraph on M1, which also names FP8 draft projections).
//
//   fast     : y[m][n] = (sum_k dec(xq[m][k]) dec(wq[n][k])) * s_m * s_n, with
//              OCP E4M3 weight codes wq and per-row scales s_n prepared
//              offline, and the per-token FP8 quantization of the bf16
//              activations (inv = 448 / max|x|, code = e4m3(x * inv), round
//              to nearest even, s_m = max|x| / 448) done inside the launch.
//   critical : y[m][n] = sum_k x[m][k] w[n][k] over bf16 x and w.
//
// Both are pure weight streams (1 or 2 bytes per weight, read once for all
// M <= 16 tokens), so the kernel is built around HBM: a persistent grid of
// one 16-wave workgroup per compute unit, each wave streaming a contiguous
// range of whole 16-row tiles, double-buffered in chunks of eight 16-byte
// loads per lane.
//
// Arithmetic.  Every E4M3 value is exactly a bf16 value, so both roles run
// on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
// a fast-role weight code pair is widened exactly by one
// v_cvt_scalef32_pk_bf16_fp8 (scale 1), and the activation codes are staged
// in LDS as the bf16 values they decode to.  The gfx950 FP8 matrix
// instruction was not used: on random codes its sums differ from the exact
// ones by up to ~1e-4 of the sum of |products|, more than fp32 accumulation
// of the same products allows.
//
// Layout.  As an MFMA B operand, lane l (row r = l % 16, K group g = l / 16)
// needs, for step j of chunk c, the 16 bytes at byte (8 c + j) 64 + 16 g of
// weight row r of its tile: 64 bytes of each of 16 rows per step.  Loaded
// that way, every 128-byte line is split over two loads, which streams
// markedly slower (and far slower still with non-temporal loads) than whole
// lines.  So steps j and j + 1 (j even) load the 128-byte segment s = 4 c +
// j / 2 of all 16 rows as two whole-line loads: X covers rows 0-7, Y rows
// 8-15, 16-byte piece p of the segment of row q going to
//     X: lane (g, r) <- row r % 8,     piece g + 4 (r / 8)
//     Y: lane (g, r) <- row 8 + r % 8, piece g + 4 (1 - r / 8).
// Then step j's operand is X where r < 8 and Y elsewhere -- row r, piece g,
// already in place -- and step j + 1's is the other of the two rotated by 8
// lanes within each 16-lane row (one DPP move): row r, piece g + 4.  The
// lane's bf16 values are elements e0 .. e0 + 7 (+ 8 .. 15 for FP8 codes, a
// second MFMA) of weight column r; the A operand of token row r reads the
// same elements of staged token row r, so the contraction covers every k
// exactly once, and lane (g, r) ends with tokens 4g .. 4g+3 of weight row r.
// Loads past the row end or past N fall outside the buffer descriptor and
// return zeros; token rows past M read a zero block.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kRawBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

constexpr int kPieceP = 512;              // activation elements per wave load pass
constexpr int kPasses = 8;                // passes: K <= 4096
constexpr int kScaleTiles = 4;            // weight-scale tiles per wave staged in LDS
static_assert(kScaleTiles * 16 == 64, "one weight scale per thread");

// Launch shape: NWV waves per workgroup, LD 16-byte weight loads per lane
// per chunk.
constexpr int kShapeWaves = 16;
constexpr int kShapeLoads = 8;
template <bool FP8, int NWV, int LD>
struct Role {
    static constexpr int kElemBytes = FP8 ? 1 : 2;
    static constexpr int kPerLoad = FP8 ? 64 : 32;  // row elements per 64-byte load step
    static constexpr int kChunk = LD * kPerLoad;
};

// LDS: M staged token rows of Kp bf16 values (stride 2 Kp + 16 bytes, so
// that the 16 token rows of one B read fall on different banks) | a 16-byte
// zero block | token scales [16] | weight scales of each wave's first
// kScaleTiles tiles [waves][kScaleTiles][16].
__host__ __device__ constexpr int stage_stride(int Kp) { return 2 * Kp + 16; }
__host__ __device__ constexpr int stage_bytes(int M, int Kp, int waves) {
    return M * stage_stride(Kp) + 16 + 16 * 4 + waves * kScaleTiles * 16 * 4;
}

// Two E4M3 codes (the low or high 16 bits of w) widened to a bf16 pair:
// every E4M3 value is a bf16 value, so the conversion (scale 1) is exact.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ v8bf as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint4 u = make_uint4(a, b, c, d);
    return __builtin_bit_cast(v8bf, u);
}

template <int LD>
__device__ __forceinline__ void load_chunk(uint4 (&buf)[LD], const uint8_t *W, int tile,
                                           int tile_end, int N, int row_bytes, int c, int r, int g) {
    static_assert(LD % 2 == 0, "loads come in X, Y pairs");
    // tiles at or past tile_end (this wave's range) load nothing
    const int n0 = tile * 16;
    const int rows = tile < tile_end ? min(16, N - n0) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(W + static_cast<int64_t>(tile < tile_end ? n0 : 0) * row_bytes), 0,
        __builtin_amdgcn_readfirstlane(rows * row_bytes), kRawBufferFlags);
    const int hi = r >> 3;
#pragma unroll
    for (int j = 0; j < LD; ++j) {
        const int seg = (c * LD + j) >> 1;
        const int row = (j & 1) ? 8 + (r & 7) : (r & 7);
        const int piece = g + 4 * ((j & 1) ? hi ^ 1 : hi);
        const int col = seg * 128 + 16 * piece;
        const uint32_t off = col < row_bytes ? static_cast<uint32_t>(row * row_bytes + col) : kOutOfRange;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kWeightPolicy);
        buf[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// The X, Y pair of loads j, j + 1 -> the operands of steps j and j + 1.
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ void unpair(uint4 &x, uint4 &y, bool lo) {
    const uint4 t0 = lo ? x : y;
    const uint4 z = lo ? y : x;
    x = t0;
    y = make_uint4(ror8(z.x), ror8(z.y), ror8(z.z), ror8(z.w));
}

template <bool FP8, int LD>
__device__ __forceinline__ v4f compute_chunk(uint4 (&buf)[LD], v4f acc, const uint8_t *bsrc,
                                             int estep, int c, int g, bool lo) {
#pragma unroll
    for (int j = 0; j < LD; j += 2)
        unpair(buf[j], buf[j + 1], lo);
#pragma unroll
    for (int j = 0; j < LD; ++j) {
        const uint4 w = buf[j];
        if constexpr (FP8) {
            const int e0 = (c * LD + j) * 64 + 16 * g;
            const v8bf a0 = as_bf16x8(fp8x2_bf16<false>(w.x), fp8x2_bf16<true>(w.x),
                                      fp8x2_bf16<false>(w.y), fp8x2_bf16<true>(w.y));
            const v8bf a1 = as_bf16x8(fp8x2_bf16<false>(w.z), fp8x2_bf16<true>(w.z),
                                      fp8x2_bf16<false>(w.w), fp8x2_bf16<true>(w.w));
            const v8bf b0 = *reinterpret_cast<const v8bf *>(bsrc + 2 * e0 * estep);
            const v8bf b1 = *reinterpret_cast<const v8bf *>(bsrc + 2 * (e0 + 8) * estep);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, a0, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, a1, acc, 0, 0, 0);
        } else {
            const int e0 = (c * LD + j) * 32 + 8 * g;
            const v8bf a = __builtin_bit_cast(v8bf, w);
            const v8bf b = *reinterpret_cast<const v8bf *>(bsrc + 2 * e0 * estep);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc, 0, 0, 0);
        }
    }
    return acc;
}

// DEFER: the workgroup gathers its outputs in LDS after the staged rows
// ([M][its rows] floats) and writes each token row's run once every wave is
// done, instead of storing tile pairs inside the weight stream (stores in
// the stream slow it far more than their bytes; the launcher picks DEFER
// where the rows fit).
template <bool FP8, int NWV, int LD, bool DEFER>
__global__ __launch_bounds__(64 * NWV) void projection_kernel(
    const uint8_t *__restrict__ W, const float *__restrict__ wscale,
    const uint16_t *__restrict__ x, int M, int K, int N, int Kp, float *__restrict__ y, int ldy,
    uint8_t *__restrict__ xq_out, float *__restrict__ xs_out) {
    using R = Role<FP8, NWV, LD>;
    constexpr int kRows = (TWD_MAX_M + NWV - 1) / NWV;  // token rows staged per wave
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int stride = stage_stride(Kp);
    uint8_t *zero = smem + M * stride;
    float *st_scale = reinterpret_cast<float *>(zero + 16);
    float *st_ws = st_scale + 16;  // [wave][kScaleTiles][16]
    const int row_bytes = K * R::kElemBytes;
    const int tiles = (N + 15) / 16;
    const int nwaves = gridDim.x * NWV;
    const int C = Kp / R::kChunk;  // chunks per tile
    // each wave owns a contiguous, even-sized range of tiles: it writes the
    // outputs of two neighbouring tiles together, so that every 128-byte
    // line of y leaves the L2 whole (a half-written line would be evicted
    // by the weight stream before its other half arrived)
    const int tpw = 2 * ((tiles + 2 * nwaves - 1) / (2 * nwaves));
    const int first = (blockIdx.x * NWV + wave) * tpw;
    const int ntiles = max(0, min(tpw, tiles - first));
    const int tile_end = first + ntiles;
    const int total = ntiles * C;
    float *ybuf = reinterpret_cast<float *>(smem + stage_bytes(M, Kp, NWV));
    const int wg_rows = NWV * tpw * 16;
    const int wg_n0 = blockIdx.x * wg_rows;

    // 1. Loads, oldest first, so that waiting for the activations never
    //    waits for weights: (fast role) one weight scale per thread -- row
    //    16 (first tile of wave tid / 64, + (tid / 16) % 4) + tid % 16 --
    //    then this wave's token row, then the first two weight chunks.
    float wsv = 0.0f;
    if constexpr (FP8) {
        const int w = tid >> 6;
        const int n = ((blockIdx.x * NWV + w) * tpw + ((tid >> 4) & 3)) * 16 + (tid & 15);
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(wscale), 0, N * 4, kRawBufferFlags);
        wsv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            sr, n < N ? static_cast<uint32_t>(4 * n) : kOutOfRange, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    // wave w stages token rows w, w + NWV, ...; lane l takes elements
    // 512 p + 8 l .. + 7 of pass p (zeros past K)
    uint4 xv[kRows][kPasses];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int m = wave + NWV * i;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(x + static_cast<int64_t>(m < M ? m : 0) * K), 0,
            __builtin_amdgcn_readfirstlane(m < M ? K * 2 : 0), kRawBufferFlags);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int k0 = kPieceP * p + 8 * lane;
            const uint32_t off = k0 < K ? static_cast<uint32_t>(2 * k0) : kOutOfRange;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            xv[i][p] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Every step issues LD loads and, unless the outputs are deferred, then
    // 8 stores (out of range, and so dropped, unless a tile pair has just
    // finished): the body is straight-line and the load counter waits stay
    // exact, one chunk always in flight.
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        y, 0, M * ldy * 4, kRawBufferFlags);
    uint4 bA[LD], bB[LD];
    int t_ld = first, c_ld = 0;  // next item to load
    auto next_load = [&](uint4 (&buf)[LD]) {
        load_chunk<LD>(buf, W, t_ld, tile_end, N, row_bytes, c_ld, r, g);
        if (++c_ld == C) {
            c_ld = 0;
            ++t_ld;
        }
    };
    // (the tile-finished condition enters as a row limit, so the stores
    // stay unconditional per-lane selects rather than a branch)
    // stores of tile pair (held, cur) at rows n and n + 16; each limit is N
    // when that tile is to be written now, else 0
    auto put = [&](v4f held, v4f cur, int n, int lim_h, int lim_c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            // (unsigned compares: n is negative for an unpaired first tile)
            const bool okh = m < M && static_cast<unsigned>(n) < static_cast<unsigned>(lim_h);
            const bool okc = m < M && static_cast<unsigned>(n + 16) < static_cast<unsigned>(lim_c);
            const uint32_t oh = okh ? static_cast<uint32_t>(4 * (m * ldy + n)) : kOutOfRange;
            const uint32_t oc = okc ? static_cast<uint32_t>(4 * (m * ldy + n + 16)) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[i]), yr, oh, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur[i]), yr, oc, 0, 0);
        }
    };
    const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    next_load(bA);
    if constexpr (!DEFER)
        put(zero4, zero4, 0, 0, 0);
    next_load(bB);
    if constexpr (!DEFER)
        put(zero4, zero4, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // 2. stage the activations as bf16 (wave w owns token rows w, w + NWV)
    if constexpr (FP8)
        st_ws[tid] = wsv;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int m = wave + NWV * i;
        if (m >= M)
            break;
        uint8_t *row = smem + m * stride;
        if constexpr (FP8) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                am2 = absmax_pair(am2, xv[i][p].x);
                am2 = absmax_pair(am2, xv[i][p].y);
                am2 = absmax_pair(am2, xv[i][p].z);
                am2 = absmax_pair(am2, xv[i][p].w);
            }
            const float a = __uint_as_float(wave_umax(absmax_bits(am2)));
            // correctly rounded fp32 divisions (build flag)
            const float inv = a > 0.0f ? 448.0f / a : 0.0f;
            const float s = a / 448.0f;
            if (lane == 0) {
                st_scale[m] = s;
                if (xs_out && blockIdx.x == 0)
                    xs_out[m] = s;
            }
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int k0 = kPieceP * p + 8 * lane;
                const uint32_t w4[4] = {xv[i][p].x, xv[i][p].y, xv[i][p].z, xv[i][p].w};
                uint32_t q[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t lo = w4[2 * h], hi = w4[2 * h + 1];
                    // x * inv rounded to fp32 on its own, then to E4M3
                    // (nearest even); an all-zero row gives +0 codes
                    const float p0 = __fmul_rn(__uint_as_float(lo << 16), inv);
                    const float p1 = __fmul_rn(__uint_as_float(lo & 0xFFFF0000u), inv);
                    const float p2 = __fmul_rn(__uint_as_float(hi << 16), inv);
                    const float p3 = __fmul_rn(__uint_as_float(hi & 0xFFFF0000u), inv);
                    const int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                    const int c0123 = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, c01, true);
                    q[h] = a > 0.0f ? static_cast<uint32_t>(c0123) : 0u;
                }
                if (xq_out && blockIdx.x == 0 && k0 < K)
                    *reinterpret_cast<uint2 *>(xq_out + static_cast<int64_t>(m) * K + k0) =
                        make_uint2(q[0], q[1]);
                if (k0 < Kp)
                    *reinterpret_cast<uint4 *>(row + 2 * k0) =
                        make_uint4(fp8x2_bf16<false>(q[0]), fp8x2_bf16<true>(q[0]),
                                   fp8x2_bf16<false>(q[1]), fp8x2_bf16<true>(q[1]));
            }
        } else {
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int k0 = kPieceP * p + 8 * lane;
                if (k0 < Kp)
                    *reinterpret_cast<uint4 *>(row + 2 * k0) = xv[i][p];
            }
        }
    }
    if (tid < 4)
        reinterpret_cast<uint32_t *>(zero)[tid] = 0u;
    __syncthreads();  // staged rows, scales, weight scales, zero block

    // 3. stream this wave's tiles: compute a chunk, then reload its buffer
    //    with the item two ahead
    const uint8_t *bsrc = r < M ? smem + r * stride : zero;
    const int estep = r < M ? 1 : 0;
    // the tokens are the MFMA's A rows and the weight rows its B columns:
    // lane (g, r) accumulates tokens 4g .. 4g+3 against weight row r, so
    // each of its four stores is one of 16 contiguous floats of a y row
    float sx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sx[i] = FP8 && 4 * g + i < M ? st_scale[4 * g + i] : 1.0f;
    int t_cp = first, c_cp = 0, ord = 0;  // item being computed, its tile ordinal
    v4f acc = zero4, held = zero4;
    auto step = [&](uint4 (&buf)[LD]) {
        acc = compute_chunk<FP8, LD>(buf, acc, bsrc, estep, c_cp, g, r < 8);
        next_load(buf);
        v4f v = acc;
        if constexpr (FP8) {
            const int o = ord < kScaleTiles ? ord : kScaleTiles - 1;
            const float ws = st_ws[(wave * kScaleTiles + o) * 16 + r];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = acc[i] * sx[i] * ws;
        }
        const bool fin = c_cp == C - 1;
        if constexpr (DEFER) {
            // rows past N are never written out
            if (fin) {
                const int row = t_cp * 16 + r - wg_n0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i < M)
                        ybuf[(4 * g + i) * wg_rows + row] = v[i];
            }
        } else {
            // a finished tile with an odd ordinal completes a pair: write
            // both; an even one waits in `held`, unless it is the wave's last
            const bool odd = (ord & 1) != 0;
            const int lim_h = fin && odd ? N : 0;
            const int lim_c = fin && (odd || ord == ntiles - 1) ? N : 0;
            const int n = (t_cp - (odd ? 1 : 0)) * 16 + r;
            put(held, v, n - (odd ? 0 : 16), lim_h, lim_c);
            if (fin && !odd)
                held = v;
        }
        if (++c_cp == C) {
            c_cp = 0;
            ++t_cp;
            ++ord;
            acc = zero4;
        }
    };
    for (int it = 0; it < total; it += 2) {
        step(bA);
        if (it + 1 >= total)
            break;
        step(bB);
    }

    // 4. deferred outputs: each token row's run of this workgroup's rows, in
    //    16-byte words where N and ldy are multiples of 4 and y is 16-byte
    //    aligned, else in 4-byte words
    if constexpr (DEFER) {
        __syncthreads();
        const int valid = min(wg_rows, N - wg_n0);
        const bool vec = ((N | ldy) & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
        for (int m = 0; m < M; ++m) {
            float *dst = y + static_cast<int64_t>(m) * ldy + wg_n0;
            const float *src = ybuf + m * wg_rows;
            if (vec) {
                for (int j = 4 * tid; j < valid; j += 4 * 64 * NWV)
                    *reinterpret_cast<v4f *>(dst + j) = *reinterpret_cast<const v4f *>(src + j);
            } else {
                for (int j = tid; j < valid; j += 64 * NWV)
                    dst[j] = src[j];
            }
        }
    }
}

using ProjFn = void (*)(const uint8_t *, const float *, const uint16_t *, int, int, int, int,
                        float *, int, uint8_t *, float *);

int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int v = cached[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64)
        cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

int projection_padded_k(bool fp8, int K) {
    const int chunk = fp8 ? Role<true, kShapeWaves, kShapeLoads>::kChunk
                          : Role<false, kShapeWaves, kShapeLoads>::kChunk;
    return (K + chunk - 1) / chunk * chunk;
}

int projection_lds_bytes(bool fp8, int M, int K) {
    return stage_bytes(M, projection_padded_k(fp8, K), kShapeWaves);
}

namespace {

// Tiles per wave as the kernel computes them for a launch of `grid`
// workgroups over `tiles` tiles.
int tiles_per_wave(int tiles, int grid) {
    const int nwaves = grid * kShapeWaves;
    return 2 * ((tiles + 2 * nwaves - 1) / (2 * nwaves));
}

}  // namespace

hipError_t launch_projection(bool fp8, const uint8_t *w, const float *wscale,
                             const uint16_t *x, int M, int K, int N, float *y,
                             uint8_t *xq_out, float *xs_out, hipStream_t stream) {
    constexpr int NWV = kShapeWaves;
    const int Kp = projection_padded_k(fp8, K);
    const int lds_stage = stage_bytes(M, Kp, NWV);
    hipError_t e = hipSuccess;
    const int cus = compute_units();
    if (cus <= 0)
        return hipErrorInvalidDevice;
    // one launch per span of rows in which every wave has at most
    // kScaleTiles tiles (the weight scales it keeps in LDS)
    const int64_t row_bytes = static_cast<int64_t>(K) * (fp8 ? 1 : 2);
    const int span = kScaleTiles * NWV * cus * 16;
    for (int n0 = 0; n0 < N; n0 += span) {
        const int rows = N - n0 < span ? N - n0 : span;
        const int tiles = (rows + 15) / 16;
        const int want = (tiles + NWV - 1) / NWV;
        const int grid = want < cus ? want : cus;
        // deferred outputs where the workgroup's rows fit beside the staging
        const int lds_defer = lds_stage + M * NWV * tiles_per_wave(tiles, grid) * 16 * 4;
        const bool defer = lds_defer <= 160 * 1024;
        const int lds = defer ? lds_defer : lds_stage;
        const ProjFn fn = fp8 ? (defer ? &projection_kernel<true, NWV, kShapeLoads, true>
                                       : &projection_kernel<true, NWV, kShapeLoads, false>)
                              : (defer ? &projection_kernel<false, NWV, kShapeLoads, true>
                                       : &projection_kernel<false, NWV, kShapeLoads, false>);
        e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * NWV), lds, stream, w + n0 * row_bytes,
                           wscale ? wscale + n0 : nullptr, x, M, K, rows, Kp, y + n0, N,
                           n0 == 0 ? xq_out : nullptr, n0 == 0 ? xs_out : nullptr);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace twd
