// VALU kernel of the W2A8 ternary linear for the narrow widths (M = 1 for
// autoregressive steps, M <= 4 for small drafted blocks), gfx950.
//
// What it computes (BitMTP page, ai.info AI summary): ternary BitNet b1.58
// weights ("What This Paper Is About"), 8-bit activations ("Main Findings":
// W2A8), and the packed low-bit operator M1 picks by replay width
// ("Methodology in Plain English", paragraph 3):
// acc[m][n] = sum_k q[m][k] t[n][k] in int32, y = acc * s_m * gamma(n).
// With FUSED the per-token absmax int8 quantization of the bf16 activations
// (same arithmetic as the stand-alone quantizer) happens inside.
//
// Work split.  A workgroup of four waves owns TW tiles of 16 weight rows and
// all of K.  Wave w takes the 256-wide K slices ("super chunks") w, w + 4,
// ..., exactly U of them (U is a compile-time count, so every load is
// straight-line code; a wave with one slice fewer loads a harmless repeat
// whose activations are zero).  Because all loads are unconditional and
// issued in order -- this wave's activation slices first, then its weights
// -- the compiler waits for the activations alone before quantizing, and for
// each weight slice only when it is consumed, so quantization and
// decode/dot overlap the weight stream.
//
// In one super chunk lane l loads 16 bytes (64 weights) of row l % 16 at K
// offset 256 s + 64 (l / 16); the whole wave covers 16 rows x 256 weights.
// Each wave stages the int8 activations of its own slices in a private LDS
// region (lane l holds elements 4l .. 4l+3 of each slice), so the only
// cross-wave synchronization is the row absmax (FUSED) and the final sum.
//
// Decode.  A 32-bit word holds 16 codes c = t + 1; masking with 0x03030303,
// 0x0C0C0C0C, 0x30303030 gives byte planes holding c, 4c, 16c for elements
// 4j..4j+3 (j = 0, 1, 2) and (w >> 6) & 0x03030303 gives plane 3.  Each
// plane is v_dot4'ed with the matching activation word into an accumulator
// per scale (x1, x4, x16), shifted back exactly at the end; sum q t =
// sum q c - sum q.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

template <int M, int U, int TW>
__host__ __device__ constexpr int act_bytes() { return kWaves * M * U * 256; }

template <int M, int U, int TW>
__host__ __device__ constexpr int red_bytes() { return M * TW * 16 * 16 * 4; }

// LDS: per-wave activation slices | partials [M][TW*16][16] | absmax
// partials [wave][M] | row-sum partials [wave][M].
template <int M, int U, int TW>
__host__ __device__ constexpr int lds_bytes() {
    return act_bytes<M, U, TW>() + red_bytes<M, U, TW>() + 2 * kWaves * M * 4;
}

template <int M, int U, int TW, bool FUSED>
__global__ __launch_bounds__(kThreads) void dot_kernel(
    const uint4 *__restrict__ W, const void *__restrict__ act,
    const float *__restrict__ xscale, int K, int N, Segments segs,
    int32_t *__restrict__ acc, float *__restrict__ y) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int CPR = K >> 6;  // 16-byte chunks per packed weight row
    const int n0 = blockIdx.x * (16 * TW);

    uint8_t *own = smem + wave * (M * U * 256);
    int32_t *red = reinterpret_cast<int32_t *>(smem + act_bytes<M, U, TW>());
    uint32_t *st_max = reinterpret_cast<uint32_t *>(smem + act_bytes<M, U, TW>() +
                                                    red_bytes<M, U, TW>());
    int32_t *st_sum = reinterpret_cast<int32_t *>(st_max + kWaves * M);

    // 1. activation loads: lane l holds elements 256 s + 4 l .. + 3 of each
    //    row for this wave's slices s = wave + 4 u (zero past K).
    bool xok[U];
    uint2 xb[FUSED ? M : 1][U];     // bf16 x 4
    uint32_t xi[FUSED ? 1 : M][U];  // int8 x 4
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k0 = 256 * (wave + kWaves * u) + 4 * lane;
        xok[u] = k0 < K;
        const int kk = xok[u] ? k0 : 0;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if constexpr (FUSED)
                xb[m][u] = *reinterpret_cast<const uint2 *>(
                    static_cast<const uint16_t *>(act) + static_cast<int64_t>(m) * K + kk);
            else
                xi[m][u] = *reinterpret_cast<const uint32_t *>(
                    static_cast<const int8_t *>(act) + static_cast<int64_t>(m) * K + kk);
        }
    }

    // 2. weight loads.  Rows past N read row N - 1 (never stored); slices
    //    past K read chunk 0 of the row (their activations are zero).
    uint4 a[U][TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int n = n0 + 16 * t + r;
        const int64_t rowbase = static_cast<int64_t>(n < N ? n : N - 1) * CPR;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kc = 4 * (wave + kWaves * u) + g;
            a[u][t] = W[rowbase + (kc < CPR ? kc : 0)];
        }
    }
    // keep every load issued before any use (the scheduler would otherwise
    // hoist activation math, and its wait, above the weight loads)
    __builtin_amdgcn_sched_barrier(0);

    // 3. own activation slices -> LDS as int8, with this wave's row sums
    int sq[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        sq[m] = 0;
    if constexpr (FUSED) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                am2 = absmax_pair(am2, xok[u] ? xb[m][u].x : 0u);
                am2 = absmax_pair(am2, xok[u] ? xb[m][u].y : 0u);
            }
            const uint32_t am = wave_umax(absmax_bits(am2));
            if (lane == 0)
                st_max[wave * M + m] = am;
        }
        __syncthreads();  // row absmax partials (LDS only)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            uint32_t am = st_max[m];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                am = max(am, st_max[w * M + m]);
            const float a_m = __uint_as_float(am);
            // correctly rounded fp32 division (build flag), as in the
            // stand-alone quantizer; an all-zero row quantizes to zeros
            const float inv = a_m > 0.0f ? 127.0f / a_m : 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t q = xok[u] ? quant4(xb[m][u].x, xb[m][u].y, inv) : 0u;
                *reinterpret_cast<uint32_t *>(own + (m * U + u) * 256 + 4 * lane) = q;
                sq[m] = sdot4(q, kOnes, sq[m]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t q = xok[u] ? xi[m][u] : 0u;
                *reinterpret_cast<uint32_t *>(own + (m * U + u) * 256 + 4 * lane) = q;
                sq[m] = sdot4(q, kOnes, sq[m]);
            }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int s = wave_sum(sq[m]);
        if (lane == 0)
            st_sum[wave * M + m] = s;
    }
    // the wave reads back only its own LDS region: its writes are ordered
    // before its reads, no workgroup barrier needed
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 4. decode + dot, one slice at a time as its weights arrive
    int d1[TW][M], d4[TW][M], d16[TW][M];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m)
            d1[t][m] = d4[t][m] = d16[t][m] = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            uint4 x[M];
#pragma unroll
            for (int m = 0; m < M; ++m)
                x[m] = *reinterpret_cast<const uint4 *>(own + (m * U + u) * 256 + 64 * g + 16 * dw);
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const uint32_t w = dw == 0 ? a[u][t].x
                                 : dw == 1 ? a[u][t].y
                                 : dw == 2 ? a[u][t].z
                                           : a[u][t].w;
                const uint32_t p0 = w & kPlane0;
                const uint32_t p1 = w & kPlane1;
                const uint32_t p2 = w & kPlane2;
                const uint32_t p3 = (w >> 6) & kPlane0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    d1[t][m] = sdot4(p0, x[m].x, d1[t][m]);
                    d4[t][m] = sdot4(p1, x[m].y, d4[t][m]);
                    d16[t][m] = sdot4(p2, x[m].z, d16[t][m]);
                    d1[t][m] = sdot4(p3, x[m].w, d1[t][m]);
                }
            }
        }
    }

    // 5. partials [M][TW*16][wave, lane group] -> LDS; one thread per output
    //    adds its 16 partials, takes off the row sum and dequantizes
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m)
            red[((m * TW + t) * 16 + r) * 16 + wave * 4 + g] =
                d1[t][m] + (d4[t][m] >> 2) + (d16[t][m] >> 4);
    __syncthreads();
    constexpr int R = TW * 16;
    for (int idx = tid; idx < M * R; idx += kThreads) {
        const int m = idx / R;
        const int n = n0 + (idx - m * R);
        if (n >= N)
            continue;
        int total = 0;
#pragma unroll
        for (int p = 0; p < 16; p += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(red + idx * 16 + p);
            total += v.x + v.y + v.z + v.w;
        }
        float scale;
        if constexpr (FUSED) {
            uint32_t am = st_max[m];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                am = max(am, st_max[w * M + m]);
            scale = __uint_as_float(am) / 127.0f;
        } else {
            scale = xscale[m];
        }
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            total -= st_sum[w * M + m];
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if (acc)
            acc[o] = total;
        if (y)
            y[o] = static_cast<float>(total) * scale * row_gamma(segs, n);
    }
}

using Fn = void (*)(const uint4 *, const void *, const float *, int, int, Segments,
                    int32_t *, float *);

template <int M, int TW, bool FUSED, int... Us>
bool pick_u(int U, Fn *fn, int *lds) {
    bool found = false;
    ((U == Us ? (*fn = &dot_kernel<M, Us, TW, FUSED>, *lds = lds_bytes<M, Us, TW>(),
                 found = true)
              : false),
     ...);
    return found;
}

template <int TW, bool FUSED>
bool pick(int M, int U, Fn *fn, int *lds) {
    switch (M) {
    case 1: return pick_u<1, TW, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
    case 2: return pick_u<2, TW, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
    case 3: return pick_u<3, TW, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
    case 4: return pick_u<4, TW, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds);
    }
    return false;
}

}  // namespace

hipError_t launch_dot(int tiles, const uint8_t *w, const void *act, bool fused,
                      const float *xscale, int M, int K, int N,
                      const Segments &segs, int32_t *acc, float *y,
                      hipStream_t stream) {
    const int S = (K + 255) / 256;
    const int U = (S + kWaves - 1) / kWaves;
    Fn fn = nullptr;
    int lds = 0;
    bool ok = false;
    switch (tiles * 2 + (fused ? 1 : 0)) {
    case 2: ok = pick<1, false>(M, U, &fn, &lds); break;
    case 3: ok = pick<1, true>(M, U, &fn, &lds); break;
    case 4: ok = pick<2, false>(M, U, &fn, &lds); break;
    case 5: ok = pick<2, true>(M, U, &fn, &lds); break;
    }
    if (!ok)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    const int grid = (N + 16 * tiles - 1) / (16 * tiles);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, stream,
                       reinterpret_cast<const uint4 *>(w), act, xscale, K, N, segs,
                       acc, y);
    return hipGetLastError();
}

}  // namespace twd
