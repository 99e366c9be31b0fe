// Matrix-core kernel of the W2A8 ternary linear for the wider verification
// widths (gfx950, v_mfma_i32_16x16x64_i8).
//
// What it computes (BitMTP page, ai.info AI summary, "Methodology in Plain
// English", paragraphs 2-3: the verifier runs the anchor plus the whole draft
// through the model, and M1 picks packed low-bit operators by replay width):
// acc[m][n] = sum_k q[m][k] t[n][k] in int32 and y = acc * s_m * gamma(n) for
// up to 16 tokens, which fill the 16 B-operand columns (zero beyond M).
//
// Work split.  A workgroup owns TW tiles of 16 weight rows and all of K.
// Four compute waves take the 256-wide K slices ("super chunks") round
// robin; in one super chunk lane l loads 16 bytes (64 weights) of row l % 16
// at K offset 256 s + 64 (l / 16) -- the A-operand layout (row = lane % 16,
// K group = lane / 16).  The four 2-bit planes of a lane's four words are the
// A operands of four MFMAs (codes, 4x codes, 16x codes, codes), each with
// its own accumulator, shifted back exactly at the end; sum q t = sum q c -
// sum q with c = t + 1.  Separate staging waves (up to eight, each with
// one or two token rows) issue the loads of all their rows at once, then
// quantize (FUSED) or copy the rows into LDS while the compute waves' weight
// loads are in flight; each wave waits only for its own loads.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

// Waves that stage activation rows, and rows per staging wave.
template <int M>
__host__ __device__ constexpr int staging_waves() { return M < 8 ? M : 8; }

template <int M>
__host__ __device__ constexpr int rows_per_stager() { return (M + staging_waves<M>() - 1) / staging_waves<M>(); }

template <int M>
__host__ __device__ constexpr int block_threads() { return 64 * (kWaves + staging_waves<M>()); }

// LDS: [activation rows | per-wave partial sums] share the first region (the
// partials are written after the last activation read), then the per-row
// sums of q and scales.
template <int M, int TW>
__host__ __device__ constexpr int act_region_bytes(int K) {
    const int act = M * (K + kPad);
    const int red = M * TW * 16 * kWaves * 4;
    return ((act > red ? act : red) + 15) & ~15;
}

template <int M, int TW>
__host__ __device__ constexpr int lds_bytes(int K) {
    return act_region_bytes<M, TW>(K) + 2 * M * 4;
}

// Staging wave: quantize (FUSED) or copy the activation rows m0, m0 + step,
// ... (RPW of them, those below M) into LDS, with their sums of q and their
// scales.  The loads of all its rows are issued first (16-byte buffer loads,
// zeros past the row), so the rows' latencies overlap; one wave covers a
// whole row, so the absmax and the sum are wave reductions.
template <bool FUSED, int RPW>
__device__ __forceinline__ void stage_rows(const void *__restrict__ act,
                                           const float *__restrict__ xscale,
                                           int m0, int step, int M, int K, int lane,
                                           uint8_t *smem, int ldsK, int32_t *st_sum,
                                           float *st_scale) {
    constexpr int kMax = 16;  // 16-byte chunks per lane and row (K <= 8192 bf16)
    constexpr int kEl = FUSED ? 2 : 1;
    const int row_bytes = K * kEl;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(act), 0, M * row_bytes, 0x00020000);
    uint4 v[RPW][kMax];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int m = m0 + step * i;
#pragma unroll
        for (int j = 0; j < kMax; ++j) {
            const int c = lane + 64 * j;
            const uint32_t off = (m < M && 16 * c < row_bytes)
                                     ? static_cast<uint32_t>(m * row_bytes + 16 * c)
                                     : 0x80000000u;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            v[i][j] = make_uint4(x[0], x[1], x[2], x[3]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int m = m0 + step * i;
        if (m >= M)
            break;  // wave-uniform
        uint8_t *dst = smem + m * ldsK;
        int part = 0;
        if constexpr (FUSED) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int j = 0; j < kMax; ++j) {
                am2 = absmax_pair(am2, v[i][j].x);
                am2 = absmax_pair(am2, v[i][j].y);
                am2 = absmax_pair(am2, v[i][j].z);
                am2 = absmax_pair(am2, v[i][j].w);
            }
            const float a = __uint_as_float(wave_umax(absmax_bits(am2)));
            // correctly rounded fp32 division (build flag), as in the
            // stand-alone quantizer; an all-zero row quantizes to zeros
            const float inv = a > 0.0f ? 127.0f / a : 0.0f;
#pragma unroll
            for (int j = 0; j < kMax; ++j) {
                const int c = lane + 64 * j;
                const uint32_t lo = quant4(v[i][j].x, v[i][j].y, inv);
                const uint32_t hi = quant4(v[i][j].z, v[i][j].w, inv);
                if (16 * c < row_bytes)
                    *reinterpret_cast<uint2 *>(dst + 8 * c) = make_uint2(lo, hi);
                part = sdot4(hi, kOnes, sdot4(lo, kOnes, part));
            }
            if (lane == 0)
                st_scale[m] = a / 127.0f;
        } else {
#pragma unroll
            for (int j = 0; j < kMax; ++j) {
                const int c = lane + 64 * j;
                if (16 * c < row_bytes)
                    *reinterpret_cast<uint4 *>(dst + 16 * c) = v[i][j];
                part = sdot4(v[i][j].w, kOnes, sdot4(v[i][j].z, kOnes,
                             sdot4(v[i][j].y, kOnes, sdot4(v[i][j].x, kOnes, part))));
            }
            if (lane == 0)
                st_scale[m] = xscale[m];
        }
        part = wave_sum(part);
        if (lane < kPad / 16)
            *reinterpret_cast<uint4 *>(dst + K + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
        if (lane == 0)
            st_sum[m] = part;
    }
}

template <int M, int TW, bool FUSED>
__global__ __launch_bounds__(block_threads<M>()) void staged_kernel(
    const uint4 *__restrict__ W, const void *__restrict__ act,
    const float *__restrict__ xscale, int32_t *__restrict__ acc, float *__restrict__ y, int K,
    int N, Segments segs) {
    constexpr int UB = kLoadsPerLane / TW;  // super chunks per batch per wave
    constexpr int NS = staging_waves<M>();
    constexpr int NT = block_threads<M>();
    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;  // tile row (A) / token column (B)
    const int g = lane >> 4;  // 64-weight group inside a super chunk
    const int CPR = K >> 6;   // 16-byte chunks per packed weight row
    const int S = (K + 255) >> 8;
    const int ldsK = K + kPad;
    const int n0 = blockIdx.x * (16 * TW);

    int32_t *st_sum = reinterpret_cast<int32_t *>(smem + act_region_bytes<M, TW>(K));
    float *st_scale = reinterpret_cast<float *>(st_sum + M);

    v4i c0[TW], c3[TW], c4[TW], c16[TW];  // accumulators per plane
#pragma unroll
    for (int t = 0; t < TW; ++t)
        c0[t] = c3[t] = c4[t] = c16[t] = v4i{0, 0, 0, 0};

    // Compute waves: weight loads right away.  Rows past N read row N - 1
    // (never stored) and chunks past K read chunk 0 of the row (their
    // activations come from the zero pad), so every load is unconditional
    // per lane and inside the weight buffer.
    const bool computes = wave < kWaves;
    const int nwave = computes && S > wave ? (S - wave + kWaves - 1) / kWaves : 0;
    int64_t rowbase[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int n = n0 + 16 * t + r;
        rowbase[t] = static_cast<int64_t>(n < N ? n : N - 1) * CPR;
    }
    uint4 a[UB][TW];
    auto issue = [&](int b) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int ui = b * UB + u;
            if (ui < nwave) {  // wave-uniform (scalar branch)
                const int kc = 4 * (wave + kWaves * ui) + g;
                const int kcc = kc < CPR ? kc : 0;
#pragma unroll
                for (int t = 0; t < TW; ++t)
                    a[u][t] = load_weight16(W + rowbase[t] + kcc);
            }
        }
    };
    if (computes) {
        issue(0);
        __builtin_amdgcn_sched_barrier(0);
    } else {
        // staging wave sw takes rows sw, sw + NS, ...
        stage_rows<FUSED, rows_per_stager<M>()>(act, xscale, wave - kWaves, NS, M, K, lane,
                                                smem, ldsK, st_sum, st_scale);
    }
    __syncthreads();  // activation rows staged

    const int nbatch = (nwave + UB - 1) / UB;  // 0 for staging waves
    for (int b = 0; b < nbatch; ++b) {
        if (b > 0)
            issue(b);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int ui = b * UB + u;
            if (ui >= nwave)
                break;
            const int s = wave + kWaves * ui;
            // groups past K read the zero pad; token columns past M read
            // row 0's zero pad
            const int off = 4 * s + g < CPR ? 256 * s + 64 * g : K;
            const int boff = r < M ? r * ldsK + off : K;
            // B operand: this lane's token over its 64-weight group;
            // B_j word d = activation word 4d + j.
            uint4 xb[4];
#pragma unroll
            for (int dw = 0; dw < 4; ++dw)
                xb[dw] = *reinterpret_cast<const uint4 *>(smem + boff + 16 * dw);
            const v4i b0 = {(int)xb[0].x, (int)xb[1].x, (int)xb[2].x, (int)xb[3].x};
            const v4i b1 = {(int)xb[0].y, (int)xb[1].y, (int)xb[2].y, (int)xb[3].y};
            const v4i b2 = {(int)xb[0].z, (int)xb[1].z, (int)xb[2].z, (int)xb[3].z};
            const v4i b3 = {(int)xb[0].w, (int)xb[1].w, (int)xb[2].w, (int)xb[3].w};
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const uint4 w = a[u][t];
                const v4i p0 = {(int)(w.x & kPlane0), (int)(w.y & kPlane0),
                                (int)(w.z & kPlane0), (int)(w.w & kPlane0)};
                const v4i p1 = {(int)(w.x & kPlane1), (int)(w.y & kPlane1),
                                (int)(w.z & kPlane1), (int)(w.w & kPlane1)};
                const v4i p2 = {(int)(w.x & kPlane2), (int)(w.y & kPlane2),
                                (int)(w.z & kPlane2), (int)(w.w & kPlane2)};
                const v4i p3 = {(int)((w.x >> 6) & kPlane0), (int)((w.y >> 6) & kPlane0),
                                (int)((w.z >> 6) & kPlane0), (int)((w.w >> 6) & kPlane0)};
                c0[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(p0, b0, c0[t], 0, 0, 0);
                c4[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(p1, b1, c4[t], 0, 0, 0);
                c16[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(p2, b2, c16[t], 0, 0, 0);
                c3[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(p3, b3, c3[t], 0, 0, 0);
            }
        }
    }

    // per-wave partial sums -> LDS (reusing the activation rows), then one
    // thread per output adds them up
    __syncthreads();  // every wave is done reading activations
    int32_t *red = reinterpret_cast<int32_t *>(smem);  // [M][TW*16][kWaves]
    if (computes) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const v4i c = c0[t] + c3[t] + (c4[t] >> 2) + (c16[t] >> 4);
            if (r < M) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[((r * TW + t) * 16 + 4 * g + i) * kWaves + wave] = c[i];
            }
        }
    }
    __syncthreads();
    constexpr int R = TW * 16;
    for (int idx = tid; idx < M * R; idx += NT) {
        const int m = idx / R;
        const int n = n0 + (idx - m * R);
        if (n >= N)
            continue;
        const int4 v = *reinterpret_cast<const int4 *>(red + idx * kWaves);
        const int total = v.x + v.y + v.z + v.w - st_sum[m];
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if (acc)
            acc[o] = total;
        if (y)
            y[o] = static_cast<float>(total) * st_scale[m] * row_gamma(segs, n);
    }
}

using Fn = void (*)(const uint4 *, const void *, const float *, int32_t *, float *, int, int,
                    Segments);

template <int TW, bool FUSED, int... Ms>
struct Table {
    static bool get(int M, int K, Fn *fn, int *lds, int *threads) {
        bool found = false;
        ((M == Ms ? (*fn = &staged_kernel<Ms, TW, FUSED>, *lds = lds_bytes<Ms, TW>(K),
                     *threads = block_threads<Ms>(), found = true)
                  : false),
         ...);
        return found;
    }
};

template <int TW, bool FUSED>
using Widths = Table<TW, FUSED, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;

}  // namespace

hipError_t launch_staged(int tiles, const uint8_t *w, const void *act, bool fused,
                       const float *xscale, int M, int K, int N,
                       const Segments &segs, int32_t *acc, float *y,
                       hipStream_t stream) {
    Fn fn = nullptr;
    int lds = 0, threads = 0;
    bool ok = false;
    switch (tiles * 2 + (fused ? 1 : 0)) {
    case 2: ok = Widths<1, false>::get(M, K, &fn, &lds, &threads); break;
    case 3: ok = Widths<1, true>::get(M, K, &fn, &lds, &threads); break;
    case 4: ok = Widths<2, false>::get(M, K, &fn, &lds, &threads); break;
    case 5: ok = Widths<2, true>::get(M, K, &fn, &lds, &threads); break;
    case 8: ok = Widths<4, false>::get(M, K, &fn, &lds, &threads); break;
    case 9: ok = Widths<4, true>::get(M, K, &fn, &lds, &threads); break;
    }
    if (!ok)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    const int grid = (N + 16 * tiles - 1) / (16 * tiles);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, stream,
                       reinterpret_cast<const uint4 *>(w), act, xscale, acc, y, K, N,
                       segs);
    return hipGetLastError();
}

}  // namespace twd
