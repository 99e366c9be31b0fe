// Tile-owner matrix-core kernel of the W2A8 ternary linear for the wider
// verification widths, gfx950.
//
// What it computes (BitMTP page, ai.info AI summary, "Methodology in Plain
// English", paragraphs 2-3: the verifier runs the anchor plus the whole draft
// through the model, and M1 picks packed low-bit operators by replay width):
// acc[m][n] = sum_k q[m][k] t[n][k] in int32 and y = acc * s_m * gamma(n) for
// up to 16 tokens, which fill the B columns of v_mfma_i32_16x16x64_i8 (zero
// beyond M).  With FUSED the per-token absmax int8 quantization of the bf16
// activations (the stand-alone quantizer's arithmetic) happens inside.
//
// Work split.  A workgroup of four waves owns 64 consecutive weight rows;
// wave w owns the 16-row tile w over all of K, so its accumulators end up
// complete: no cross-wave reduction.  The activation block (M x K) is staged
// once per workgroup -- every thread loads, and with FUSED quantizes, a share
// of it into LDS -- so the quantization work per weight row is a quarter of
// what a 16-row workgroup would spend.  All weight loads of a wave (U
// 256-wide slices, a compile-time count) are issued before the staging
// starts and consumed in order.
//
// Layouts.  The A operand of slice u is, in lane (r = lane % 16, g = lane /
// 16), the 16 bytes of tile row r at K offset 256 u + 64 g.  Loaded that way
// every 128-byte line of a row would be split over two loads, so each pair
// of slices is loaded as whole lines instead (two loads: rows 0-7, rows
// 8-15) and a per-lane select plus one DPP rotation by 8 lanes rebuilds the
// two A operands; measured on the 2B gate/up shape at M = 2 and 4 this
// takes a cold launch from 5.36 to 4.91 us and 5.32 to 4.88 us.  The
// four byte planes of its four words (masks 0x03030303, 0x0C0C0C0C,
// 0x30303030 and (w >> 6) & 0x03030303: codes c = t + 1 scaled by 1, 4, 16,
// 1) are the A operands of four MFMAs with their own accumulators, shifted
// back exactly at the end; sum q t = sum q c - sum q.  Plane j of word d
// holds elements 64 g + 16 d + 4 j + b, so the matching B operand is the four
// activation words 16 g + 4 d + j (d = 0..3): the staged rows are stored with
// word 16 g + 4 d + j at position 16 g + 4 j + d, and one 16-byte LDS read
// gives a B operand.  Token columns at or past M read a zero block.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

constexpr int kRawBufferFlags = 0x00020000;  // raw buffer, 32-bit format
constexpr uint32_t kOutOfRange = 0x80000000u;

// LDS layout: staged rows [MB][U * 256 + 16] | zero block (64 B) | absmax
// partials [16][MB] | row-sum partials [16][MB] (one per wave and 16-lane
// DPP row) | scales [MB].  The 16-byte row padding puts
// the 16 token rows a B-operand read touches on 16 different 4-bank groups
// (64 banks of 4 bytes).
template <int U>
__host__ __device__ constexpr int row_stride() { return U * 256 + 16; }

template <int MB, int U>
__host__ __device__ constexpr int lds_bytes() {
    return MB * row_stride<U>() + 64 + 2 * 4 * kWaves * MB * 4 + MB * 4;
}

// Words (4 elements) of one staged row handled per thread.
template <int U>
__host__ __device__ constexpr int stage_words() { return (U * 64 + kThreads - 1) / kThreads; }

// Rotate a value by 8 lanes within each 16-lane row (DPP row_ror:8).
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false));
}

__device__ __forceinline__ int permuted_word(int w) {
    // word 16 g + 4 d + j of a slice -> 16 g + 4 j + d
    return (w & ~63) | (w & 48) | ((w & 3) << 2) | ((w >> 2) & 3);
}

template <int MB, int U, bool FUSED>
__global__ __launch_bounds__(kThreads) void tile_kernel(
    const uint8_t *__restrict__ W, const void *__restrict__ act,
    const float *__restrict__ xscale, int32_t *__restrict__ acc, float *__restrict__ y, int M,
    int K, int N, Segments segs) {
    constexpr int S = row_stride<U>();  // staged row stride
    constexpr int VW = stage_words<U>();
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *xs = smem;                 // [MB][S]
    uint8_t *zero = smem + MB * S;      // 64 zero bytes
    uint32_t *st_max = reinterpret_cast<uint32_t *>(zero + 64);         // [16][MB]
    int32_t *st_sum = reinterpret_cast<int32_t *>(st_max + 4 * kWaves * MB);  // [16][MB]
    float *st_scale = reinterpret_cast<float *>(st_sum + 4 * kWaves * MB);    // [MB]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int row_bytes = K >> 2;
    const int part = wave * 4 + (lane >> 4);  // this lane's DPP row in the workgroup

    // 1. activation loads: thread t takes words t, t + 256, ... of each of
    //    the M rows (zeros past K; rows past M are never read)
    //    Each token row has a descriptor of its own (scalar work), so one
    //    vector offset per word serves every row and the range check ends
    //    each row at K.
    constexpr int kEl = FUSED ? 2 : 1;
    const int xrow = K * kEl;
    const uint8_t *xbase = static_cast<const uint8_t *>(act);
    uint32_t xoff[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) {
        const int k0 = 4 * (tid + kThreads * v);
        xoff[v] = k0 < K ? static_cast<uint32_t>(k0 * kEl) : kOutOfRange;
    }
    uint2 xb[FUSED ? MB : 1][VW];
    uint32_t xi[FUSED ? 1 : MB][VW];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(xbase + m * xrow), 0, xrow, kRawBufferFlags);
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            const uint32_t off = xoff[v];
            if constexpr (FUSED) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0);
                xb[m][v] = make_uint2(x[0], x[1]);
            } else {
                xi[m][v] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
            }
        }
    }

    // 2. weight loads of this wave's tile; rows past N fall outside the
    //    descriptor and K groups past the row end get an out-of-range offset
    const int n_t = blockIdx.x * 64 + wave * 16;
    const int wbytes = __builtin_amdgcn_readfirstlane(max(0, min(16, N - n_t)) * row_bytes);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(W + static_cast<int64_t>(min(n_t, N - 1)) * row_bytes), 0,
        wbytes, kRawBufferFlags);
    // Slices 2p and 2p + 1 are the 128-byte segment p of each tile row: two
    // loads read it as whole lines, X rows 0-7 and Y rows 8-15, lane (g, r)
    // taking 16-byte piece g + 4 (r / 8) (X) or g + 4 (1 - r / 8) (Y) of
    // row r % 8 (X) or 8 + r % 8 (Y).  A last odd slice is loaded alone, in
    // the A layout.
    uint4 a[U];
    const int hi = r >> 3;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int row = r, col = 64 * u + 16 * g;
        if (u + 1 < U || (U & 1) == 0) {
            const int seg = 128 * (u >> 1);
            row = (u & 1) ? 8 + (r & 7) : (r & 7);
            col = seg + 16 * (g + 4 * ((u & 1) ? 1 - hi : hi));
        }
        const uint32_t off = col < row_bytes ? static_cast<uint32_t>(row * row_bytes + col)
                                             : kOutOfRange;
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kWeightPolicy);
        a[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the segment scales of the lane's four rows and the output pointers:
    // their kernel-argument loads wait here, in the shadow of the
    // activation loads
    float gam[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gam[i] = row_gamma(segs, n_t + 4 * g + i);
        settle_v(gam[i]);
    }
    settle_s(acc);
    settle_s(y);
    __builtin_amdgcn_sched_barrier(0);

    // 3. stage the M rows as int8 in the B layout, with the row sums of q
    if (tid < 16)
        reinterpret_cast<uint32_t *>(zero)[tid] = 0u;
    int sq[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
        sq[m] = 0;
    if constexpr (FUSED) {
        // row absmax: per-lane partials, reduced over each DPP row for all
        // rows at once, 16 partials per row to LDS
        uint32_t amv[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                am2 = absmax_pair(am2, xb[m][v].x);
                am2 = absmax_pair(am2, xb[m][v].y);
            }
            amv[m] = absmax_bits(am2);
        }
        row_max16<MB>(amv);
        if ((lane & 15) == 15) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                st_max[part * MB + m] = amv[m];
        }
        __syncthreads();  // absmax partials
        // lane m combines row m and divides once for it (correctly rounded
        // fp32 division, build flag, as in the stand-alone quantizer; an
        // all-zero row quantizes to zeros)
        uint32_t am_l = 0;
        if (lane < MB) {
#pragma unroll
            for (int i = 0; i < 4 * kWaves; ++i)
                am_l = max(am_l, st_max[i * MB + lane]);
        }
        const float a_l = __uint_as_float(am_l);
        const float inv_l = a_l > 0.0f ? 127.0f / a_l : 0.0f;
        if (wave == 0 && lane < MB)
            st_scale[lane] = a_l / 127.0f;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), m));
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const int word = tid + kThreads * v;
                const uint32_t q = quant4(xb[m][v].x, xb[m][v].y, inv);
                if (VW * kThreads == U * 64 || word < U * 64)
                    *reinterpret_cast<uint32_t *>(xs + m * S + 4 * permuted_word(word)) = q;
                sq[m] = sdot4(q, kOnes, sq[m]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const int word = tid + kThreads * v;
                if (VW * kThreads == U * 64 || word < U * 64)
                    *reinterpret_cast<uint32_t *>(xs + m * S + 4 * permuted_word(word)) = xi[m][v];
                sq[m] = sdot4(xi[m][v], kOnes, sq[m]);
            }
    }
    row_sum16<MB>(sq);
    if ((lane & 15) == 15) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
            st_sum[part * MB + m] = sq[m];
    }
    __syncthreads();  // staged rows, row sums

    // the epilogue's other inputs (row sum of q and scale of token r),
    // settled while weights are in flight
    int qsum = 0;
    float scale = 0.0f;
    if (r < MB) {
#pragma unroll
        for (int i = 0; i < 4 * kWaves; ++i)
            qsum += st_sum[i * MB + r];
        scale = FUSED ? st_scale[r] : xscale[r];
    }
    settle_v(qsum);
    settle_v(scale);
    __builtin_amdgcn_sched_barrier(0);

    // 4. decode + MFMA, one slice at a time as its weights arrive
    v4i c0 = {0, 0, 0, 0}, c3 = c0, c4 = c0, c16 = c0;
    const uint8_t *bsrc = r < MB ? xs + r * S + 64 * g : zero;
    const int ustep = r < MB ? 256 : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint8_t *bu = bsrc + u * ustep;
        const v4i b0 = *reinterpret_cast<const v4i *>(bu);
        const v4i b1 = *reinterpret_cast<const v4i *>(bu + 16);
        const v4i b2 = *reinterpret_cast<const v4i *>(bu + 32);
        const v4i b3 = *reinterpret_cast<const v4i *>(bu + 48);
        // operand of slice u (row r, piece g of its 64 bytes): for the first
        // slice of a pair X where r < 8, else Y; for the second, the other
        // load moved 8 lanes along the 16-lane row (row r, piece g + 4)
        uint4 au = a[u];
        if (u + 1 < U || (U & 1) == 0) {
            const uint4 x = a[u & ~1], yv = a[u | 1];
            if ((u & 1) == 0) {
                au = hi ? yv : x;
            } else {
                const uint4 z = hi ? x : yv;
                au = make_uint4(ror8(z.x), ror8(z.y), ror8(z.z), ror8(z.w));
            }
        }
        const v4i w = {static_cast<int>(au.x), static_cast<int>(au.y),
                       static_cast<int>(au.z), static_cast<int>(au.w)};
        const v4i p0 = w & static_cast<int>(kPlane0);
        const v4i p1 = w & static_cast<int>(kPlane1);
        const v4i p2 = w & static_cast<int>(kPlane2);
        const v4i p3 = (w >> 6) & static_cast<int>(kPlane0);
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p0, b0, c0, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p1, b1, c4, 0, 0, 0);
        c16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p2, b2, c16, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p3, b3, c3, 0, 0, 0);
    }

    // 5. lane (token r, group g) holds rows 4g .. 4g+3 of the tile for token
    //    r: take off the row sum, dequantize, store
    if (r < MB) {
        const v4i c = c0 + c3 + (c4 >> 2) + (c16 >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n_t + 4 * g + i;
            if (n < N) {
                const int total = c[i] - qsum;
                const int64_t o = static_cast<int64_t>(r) * N + n;
                if (acc)
                    acc[o] = total;
                if (y)
                    y[o] = static_cast<float>(total) * scale * gam[i];
            }
        }
    }
}

using Fn = void (*)(const uint8_t *, const void *, const float *, int32_t *, float *, int, int,
                    int, Segments);

template <int MB, bool FUSED, int... Us>
bool pick_u(int U, Fn *fn, int *lds) {
    bool found = false;
    ((U == Us ? (*fn = &tile_kernel<MB, Us, FUSED>, *lds = lds_bytes<MB, Us>(), found = true)
              : false),
     ...);
    return found;
}

// One instance per width: the kernel stages and quantizes exactly M token
// rows (a rounded-up block would spend VALU time on zero rows, and with one
// wave per SIMD that time is on the critical path).
template <bool FUSED, int... Ms>
bool pick_m(int M, int U, Fn *fn, int *lds) {
    bool found = false;
    ((M == Ms ? (found = pick_u<Ms, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12>(U, fn, lds))
              : false),
     ...);
    return found;
}

template <bool FUSED>
bool pick(int M, int U, Fn *fn, int *lds) {
    return pick_m<FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(M, U, fn, lds);
}

}  // namespace

bool tile_supported(int M, int K) {
    return M >= 1 && M <= TWD_MAX_M && K >= 1 && (K + 255) / 256 <= 12;
}

hipError_t launch_tile(const uint8_t *w, const void *act, bool fused, const float *xscale,
                       int M, int K, int N, const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream) {
    const int U = (K + 255) / 256;
    Fn fn = nullptr;
    int lds = 0;
    const bool ok = fused ? pick<true>(M, U, &fn, &lds) : pick<false>(M, U, &fn, &lds);
    if (!ok)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, dim3((N + 63) / 64), dim3(kThreads), lds, stream, w, act, xscale,
                       acc, y, M, K, N, segs);
    return hipGetLastError();
}

}  // namespace twd
