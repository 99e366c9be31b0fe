// Row-owner VALU kernel of the W2A8 ternary linear for the narrowest widths
// (M = 1 autoregressive steps, up to M = 4), gfx950.
//
// What it computes (BitMTP page, ai.info AI summary): ternary BitNet b1.58
// weights ("What This Paper Is About"), 8-bit activations ("Main Findings":
// W2A8), and the packed low-bit operator M1 picks by replay width
// ("Methodology in Plain English", paragraph 3):
// acc[m][n] = sum_k q[m][k] t[n][k] in int32, y = acc * s_m * gamma(n).
// With FUSED the per-token absmax int8 quantization of the bf16 activations
// (same arithmetic as the stand-alone quantizer) happens inside.
//
// Work split.  Each wave owns R whole weight rows; a workgroup of NW waves
// owns NW R consecutive rows.  L = 64 / R lanes share a row: in load u, lane
// (row r = lane / L, part p = lane % L) reads the 16 bytes at byte offset
// 16 (u L + p) of its row, so one load instruction covers L x 16 bytes of
// each of its R rows -- whole 128-byte lines.  Each wave holds all U loads of
// its lanes in flight at once (U = ceil(K / (64 L)), a compile-time count);
// loads past the row end are given an out-of-range buffer offset and return
// zeros.  The workgroup first quantizes (FUSED) or copies the activation
// rows into LDS together -- every wave needs all of K -- while the weight
// loads are in flight.  A row's partial sums are then combined with DPP row
// shifts inside the wave: no cross-wave reduction, no partials in LDS and no
// barrier after the loads; the last lane of each row group writes y.
//
// Decode as in the other linear kernels: a 32-bit word holds 16 codes
// c = t + 1; the masks 0x03030303, 0x0C0C0C0C, 0x30303030 and
// (w >> 6) & 0x03030303 give byte planes (c, 4c, 16c, c) for elements 4j..4j+3
// of the word, each v_dot4'ed with the matching activation word into an
// accumulator per scale.  Every product in the x4 (x16) accumulator is a
// multiple of 4 (16), so each lane shifts them back exactly before the
// cross-lane sum; sum q t = sum q c - sum q.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

constexpr int kRawBufferFlags = 0x00020000;  // raw buffer, 32-bit format
constexpr uint32_t kOutOfRange = 0x80000000u;

template <int R>
__host__ __device__ constexpr int lanes_per_row() { return 64 / R; }

// Activation row length: all U loads' worth of K, zero past K.  In LDS,
// 16 bytes of padding follow every 256 bytes (four 64-element chunks), so
// that the 16-byte reads of the lanes of a row group, 64 bytes apart, fall
// on different banks.
template <int R, int U>
__host__ __device__ constexpr int act_len() { return U * lanes_per_row<R>() * 64; }

template <int R, int U>
__host__ __device__ constexpr int act_stride() { return act_len<R, U>() + act_len<R, U>() / 16; }

// LDS byte offset of activation byte k of a staged row.
__device__ __forceinline__ int act_off(int k) { return k + ((k >> 8) << 4); }

// Staging: each of the NW * 64 threads quantizes / copies the 4-element
// words t, t + 64 NW, ...
template <int R, int NW, int U>
__host__ __device__ constexpr int stage_words() { return (act_len<R, U>() / 4 + 64 * NW - 1) / (64 * NW); }

template <int M, int R, int NW, int U>
__host__ __device__ constexpr int lds_bytes() { return M * act_stride<R, U>() + 2 * NW * M * 4; }

// Sum over the L lanes of each row group; the total lands in the group's
// last lane.  L = 16: row_shr 1, 2, 4, 8 within a DPP row; L = 8: row_shr
// 1, 2, 4 (a window of 8 lanes never crosses into the neighbouring group at
// lanes 7 and 15).
template <int L>
__device__ __forceinline__ int group_sum(int v) {
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    if constexpr (L == 16)
        v += dpp<0x118>(v);
    return v;
}

template <int M, int R, int NW, int U, bool FUSED>
__global__ __launch_bounds__(64 * NW) void rows_kernel(
    const uint8_t *__restrict__ W, const void *__restrict__ act,
    const float *__restrict__ xscale, int32_t *__restrict__ acc, float *__restrict__ y, int K,
    int N, Segments segs) {
    constexpr int L = lanes_per_row<R>();
    constexpr int S = act_stride<R, U>();  // LDS row stride
    constexpr int SL = act_len<R, U>();    // staged elements per row
    constexpr int V = stage_words<R, NW, U>();
    constexpr int T = 64 * NW;
    static_assert(L == 8 || L == 16, "row groups of 8 or 16 lanes");
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *xs = smem;  // [M][S] int8
    uint32_t *st_max = reinterpret_cast<uint32_t *>(smem + M * S);
    int32_t *st_sum = reinterpret_cast<int32_t *>(st_max + NW * M);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane / L;
    const int p = lane % L;
    const int n0 = blockIdx.x * (NW * R);
    const int row_bytes = K >> 2;

    // 1. activation loads for the cooperative staging: thread t takes the
    //    4-element words t, t + T, ... of every row (zeros past K)
    constexpr int kEl = FUSED ? 2 : 1;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(act), 0, M * K * kEl, kRawBufferFlags);
    uint2 xb[FUSED ? M : 1][V];
    uint32_t xi[FUSED ? 1 : M][V];
    //    (U = ceil(K / (64 L)) puts every word of the first V - 1 rounds
    //    below K: only the last round needs the range test)
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int k0 = 4 * (tid + T * v);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint32_t off = (v < V - 1 || k0 < K)
                                     ? static_cast<uint32_t>((m * K + k0) * kEl)
                                     : kOutOfRange;
            if constexpr (FUSED) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0);
                xb[m][v] = make_uint2(x[0], x[1]);
            } else {
                xi[m][v] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
            }
        }
    }

    // 2. weight loads: this wave's R rows; past the row end -> zeros
    const int n_wave = n0 + wave * R;
    // (wave-uniform; readfirstlane keeps the descriptor in scalar registers)
    const int wbytes = __builtin_amdgcn_readfirstlane(max(0, min(R, N - n_wave)) * row_bytes);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(W + static_cast<int64_t>(min(n_wave, N - 1)) * row_bytes), 0,
        wbytes, kRawBufferFlags);
    //    (likewise only the last load can pass the row end)
    uint4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int col = 16 * (u * L + p);
        const uint32_t off = (u < U - 1 || col < row_bytes)
                                 ? static_cast<uint32_t>(r * row_bytes + col)
                                 : kOutOfRange;
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kWeightPolicy);
        a[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the segment scale of this lane's row and the output pointers: their
    // kernel-argument loads wait here, in the shadow of the activation loads
    const int n = n_wave + r;
    float gam = row_gamma(segs, n);
    settle_v(gam);
    settle_s(acc);
    settle_s(y);
    __builtin_amdgcn_sched_barrier(0);

    // 3. stage the activation rows as int8 (with the row sums of q).
    //    Everything the epilogue needs besides the dot products -- scales,
    //    row sums of q, the segment scale of this lane's row -- is settled
    //    here, while the weights are still in flight.
    float scale[M];
    if constexpr (!FUSED) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            scale[m] = xscale[m];
    }
    int sq[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        sq[m] = 0;
    if constexpr (FUSED) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int v = 0; v < V; ++v) {
                am2 = absmax_pair(am2, xb[m][v].x);
                am2 = absmax_pair(am2, xb[m][v].y);
            }
            const uint32_t am = wave_umax(absmax_bits(am2));
            if (lane == 0)
                st_max[wave * M + m] = am;
        }
        __syncthreads();  // absmax partials
#pragma unroll
        for (int m = 0; m < M; ++m) {
            uint32_t am = st_max[m];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                am = max(am, st_max[w * M + m]);
            const float a_m = __uint_as_float(am);
            // correctly rounded fp32 divisions (build flag), as in the
            // stand-alone quantizer; an all-zero row quantizes to zeros
            const float inv = a_m > 0.0f ? 127.0f / a_m : 0.0f;
            scale[m] = a_m / 127.0f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int word = tid + T * v;
                const uint32_t q = quant4(xb[m][v].x, xb[m][v].y, inv);
                if (V * T * 4 == SL || 4 * word < SL)
                    *reinterpret_cast<uint32_t *>(xs + m * S + act_off(4 * word)) = q;
                sq[m] = sdot4(q, kOnes, sq[m]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int word = tid + T * v;
                if (V * T * 4 == SL || 4 * word < SL)
                    *reinterpret_cast<uint32_t *>(xs + m * S + act_off(4 * word)) = xi[m][v];
                sq[m] = sdot4(xi[m][v], kOnes, sq[m]);
            }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int s = wave_sum(sq[m]);
        if (lane == 0)
            st_sum[wave * M + m] = s;
    }
    __syncthreads();  // staged rows and row sums
    int qsum[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        qsum[m] = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            qsum[m] += st_sum[w * M + m];
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
        settle_v(scale[m]);
    __builtin_amdgcn_sched_barrier(0);

    // 4. decode + dot, one load at a time as it arrives.  The x1, x4 and
    //    x16 sums run over all loads and are combined once: every term of
    //    d4 (d16) is a multiple of 4 (16), so the shifts are exact, and
    //    |d16| <= 16 * 2 * 127 * K / 4 < 2^31 for K <= 8192.
    //    Where they fit in registers (M U <= 8), the staged activation words
    //    of every load are read from LDS right after the barrier, so their
    //    latency passes while the weights are awaited instead of after each
    //    weight load lands.
    constexpr bool kPre = M * U <= 8;
    uint4 xa[kPre ? U : 1][kPre ? M : 1][4];
    if constexpr (kPre) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int dw = 0; dw < 4; ++dw)
                    xa[u][m][dw] = *reinterpret_cast<const uint4 *>(
                        xs + m * S + act_off(64 * (u * L + p)) + 16 * dw);
        __builtin_amdgcn_sched_barrier(0);
    }
    int d1[M], d4[M], d16[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        d1[m] = d4[m] = d16[m] = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int kb = act_off(64 * (u * L + p));  // first element of this chunk
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            const uint32_t w = dw == 0 ? a[u].x : dw == 1 ? a[u].y : dw == 2 ? a[u].z : a[u].w;
            const uint32_t p0 = w & kPlane0;
            const uint32_t p1 = w & kPlane1;
            const uint32_t p2 = w & kPlane2;
            const uint32_t p3 = (w >> 6) & kPlane0;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 x = kPre ? xa[kPre ? u : 0][kPre ? m : 0][dw]
                                     : *reinterpret_cast<const uint4 *>(xs + m * S + kb + 16 * dw);
                d1[m] = sdot4(p0, x.x, d1[m]);
                d4[m] = sdot4(p1, x.y, d4[m]);
                d16[m] = sdot4(p2, x.z, d16[m]);
                d1[m] = sdot4(p3, x.w, d1[m]);
            }
        }
    }
    int tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        tot[m] = d1[m] + (d4[m] >> 2) + (d16[m] >> 4);

    // 5. row totals across the row group; its last lane writes the outputs
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int t = group_sum<L>(tot[m]) - qsum[m];
        if (p == L - 1 && n < N) {
            const int64_t o = static_cast<int64_t>(m) * N + n;
            if (acc)
                acc[o] = t;
            if (y)
                y[o] = static_cast<float>(t) * scale[m] * gam;
        }
    }
}

using Fn = void (*)(const uint8_t *, const void *, const float *, int32_t *, float *, int, int,
                    Segments);

template <int M, int R, int NW, bool FUSED, int... Us>
bool pick_u(int U, Fn *fn, int *lds) {
    bool found = false;
    ((U == Us ? (*fn = &rows_kernel<M, R, NW, Us, FUSED>, *lds = lds_bytes<M, R, NW, Us>(),
                 found = true)
              : false),
     ...);
    return found;
}

// U = ceil(K / (64 L)) <= 8 (R = 4) or 16 (R = 8) for K <= 8192.  The
// shapes with 8 rows per wave (wide outputs) exist for M <= 2; M = 3, 4 take
// 4 rows per wave and four waves.
template <bool FUSED>
bool pick(int M, int R, int NW, int U, Fn *fn, int *lds) {
    if (R == 4 && NW == 4) {
        switch (M) {
        case 1: return pick_u<1, 4, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
        case 2: return pick_u<2, 4, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
        case 3: return pick_u<3, 4, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
        case 4: return pick_u<4, 4, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
        }
        return false;
    }
    if (M > 2 || R != 8)
        return false;
    if (M == 1 && NW == 4)
        return pick_u<1, 8, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(U, fn, lds);
    if (M == 1 && NW == 8)
        return pick_u<1, 8, 8, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(U, fn, lds);
    if (M == 2 && NW == 4)
        return pick_u<2, 8, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(U, fn, lds);
    if (M == 2 && NW == 8)
        return pick_u<2, 8, 8, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(U, fn, lds);
    return false;
}

}  // namespace

// Rows per workgroup from the output size: the most (64, 32, then 16) that
// still leaves about one workgroup per compute unit -- fewer workgroups
// quantize the activations fewer times, but under ~200 of them the loads in
// flight no longer fill the chip.  Measured on the 2B shapes at M = 1.
void rows_shape(int M, int K, int N, int *rows_per_wave, int *waves) {
    *rows_per_wave = 4;
    *waves = 4;
    // 8 rows per wave at M = 2 holds 8 or more loads per lane past K = 3584,
    // more than the registers of two waves per SIMD: those shapes would spill
    if (M > 2 || (M == 2 && K > 7 * 512))
        return;
    if (N / 64 >= 200) {
        *rows_per_wave = 8;
        *waves = 8;
    } else if (N / 32 >= 200) {
        *rows_per_wave = 8;
        *waves = 4;
    }
}

hipError_t launch_rows(const uint8_t *w, const void *act, bool fused, const float *xscale,
                       int M, int K, int N, const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream) {
    int R = 4, NW = 4;
    rows_shape(M, K, N, &R, &NW);
    const int L = 64 / R;
    const int U = (K + 64 * L - 1) / (64 * L);
    Fn fn = nullptr;
    int lds = 0;
    const bool ok = fused ? pick<true>(M, R, NW, U, &fn, &lds) : pick<false>(M, R, NW, U, &fn, &lds);
    if (!ok)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    const int per_block = NW * R;
    hipLaunchKernelGGL(fn, dim3((N + per_block - 1) / per_block), dim3(64 * NW), lds, stream,
                       w, act, xscale, acc, y, K, N, segs);
    return hipGetLastError();
}

}  // namespace twd
