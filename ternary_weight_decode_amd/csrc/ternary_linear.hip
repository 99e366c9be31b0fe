// W2A8 ternary linear kernels for gfx950 (CDNA4).
//
// What they compute (BitMTP page, ai.info AI summary): the packed low-bit
// operators that M1 selects "by replay width and input/output dimensions"
// ("Methodology in Plain English", paragraph 3), with ternary weights
// ("What This Paper Is About") and W2A8 = 2-bit weights, 8-bit activations
// ("Main Findings"):  acc[m][n] = sum_k q[m][k] * t[n][k] in int32 and
// y[m][n] = acc[m][n] * s_m * gamma(n).
//
// Work split.  A workgroup owns TW tiles of 16 consecutive weight rows and
// the whole K range; its four waves take the 256-wide K slices ("super
// chunks") round robin.  In one super chunk, lane l loads 16 bytes -- 64
// weights -- of row (l % 16) at K offset 256 s + 64 (l / 16), so a wave-wide
// load covers 16 rows x 256 weights = 1 KiB and every row segment is 64
// contiguous bytes.  The same lane mapping is the A-operand layout of
// v_mfma_i32_16x16x64_i8 (row = lane % 16, K group = lane / 16), so both
// kernel families share the loads and the workgroup skeleton:
//   1. issue the first batch of weight loads (they depend on nothing),
//   2. copy the M int8 activation rows into LDS and sum each row,
//   3. decode + multiply-accumulate, batch by batch,
//   4. reduce the four waves' partials through LDS and write acc / y.
//
// Decode.  A 32-bit word holds 16 codes c = t + 1; masking it with
// 0x03030303, 0x0C0C0C0C and 0x30303030 gives three byte planes holding
// c, 4c and 16c for elements 4j..4j+3 (j = 0, 1, 2), and (w >> 6) & 0x03030303
// gives plane 3.  Each plane lines up with one word of int8 activations, so
// no shuffle is needed; the planes scaled by 4 and 16 go to their own
// accumulators, which are shifted back exactly at the end.  Since c = t + 1,
// sum q t = sum q c - sum q, and the row sums of q come from step 2.
//
//   DOT  (VALU): v_dot4 of each plane with the activation word, per token.
//   MFMA (matrix cores): the four planes of a lane's four words form the A
//        operands of four 16x16x64 int8 MFMAs; tokens fill the 16 B columns
//        (zero beyond M).
#include <atomic>

#include "twd_internal.h"

namespace twd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLoadsPerLane = 8;  // 16-byte weight loads in flight per lane

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kPlane0 = 0x03030303u;
constexpr uint32_t kPlane1 = 0x0C0C0C0Cu;  // codes x 4
constexpr uint32_t kPlane2 = 0x30303030u;  // codes x 16
constexpr uint32_t kOnes = 0x01010101u;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c,
                                  false);
}

__device__ __forceinline__ int byte_sum(const uint4 v, int c) {
    c = sdot4(v.x, kOnes, c);
    c = sdot4(v.y, kOnes, c);
    c = sdot4(v.z, kOnes, c);
    return sdot4(v.w, kOnes, c);
}

__device__ __forceinline__ float row_gamma(const Segments &sg, int n) {
    float g = sg.gamma[0];
#pragma unroll
    for (int s = 1; s < TWD_MAX_SEGMENTS; ++s)
        if (s < sg.nseg && n >= sg.bound[s - 1])
            g = sg.gamma[s];
    return g;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Activation rows in LDS are K bytes of data followed by kPad zero bytes:
// lanes whose 64-weight group lies past K (a partial last super chunk) and
// MFMA token columns past M read the zeros, so out-of-range work adds
// nothing and no load needs a per-lane branch.  The extra 16 bytes spread
// consecutive token rows over the LDS banks.
constexpr int kPad = 80;

// LDS bytes for the activation rows (also reused for the partial sums once
// the main loop is done), rounded to 16.
__host__ __device__ constexpr int act_region_bytes(int M, int K, int TW) {
    const int act = M * (K + kPad);
    const int red = kWaves * M * TW * 16 * 4;
    const int r = act > red ? act : red;
    return (r + 15) & ~15;
}

template <int M, int TW>
__host__ __device__ constexpr int lds_bytes(int K) {
    return act_region_bytes(M, K, TW) + kWaves * M * 4;
}

template <int KERNEL, int M, int TW>
__global__ __launch_bounds__(kThreads) void linear_kernel(
    const uint4 *__restrict__ W, const int8_t *__restrict__ xq,
    const float *__restrict__ xscale, int K, int N, Segments segs,
    int32_t *__restrict__ acc, float *__restrict__ y) {
    constexpr int UB = kLoadsPerLane / TW;  // super chunks per batch per wave
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
    const int nwave = S > wave ? (S - wave + kWaves - 1) / kWaves : 0;

    int32_t *sq_part = reinterpret_cast<int32_t *>(smem + act_region_bytes(M, K, TW));

    // Row bases of this lane's tiles.  Rows past N read row N - 1 (the
    // results of those rows are never stored) and chunks past K read chunk 0
    // of the row (their activations come from the zero pad), so every load
    // is unconditional and stays inside the weight buffer.
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
                    a[u][t] = W[rowbase[t] + kcc];
            }
        }
    };

    // 1. first batch of weight loads
    issue(0);

    // 2. activations -> LDS, row sums of q
    {
        const int c16 = K >> 4;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xq + static_cast<int64_t>(m) * K);
            int part = 0;
            for (int c = tid; c < c16; c += kThreads) {
                const uint4 v = src[c];
                *reinterpret_cast<uint4 *>(smem + m * ldsK + 16 * c) = v;
                part = byte_sum(v, part);
            }
            if (tid < kPad / 16)
                *reinterpret_cast<uint4 *>(smem + m * ldsK + K + 16 * tid) =
                    make_uint4(0u, 0u, 0u, 0u);
            part = wave_sum(part);
            if (lane == 0)
                sq_part[wave * M + m] = part;
        }
    }
    __syncthreads();

    // 3. main loop
    int d1[TW][M], d4[TW][M], d16[TW][M];  // DOT accumulators (x1, x4, x16)
    v4i c0[TW], c3[TW], c4[TW], c16[TW];    // MFMA accumulators per plane
#pragma unroll
    for (int t = 0; t < TW; ++t) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            d1[t][m] = d4[t][m] = d16[t][m] = 0;
        c0[t] = c3[t] = c4[t] = c16[t] = v4i{0, 0, 0, 0};
    }

    const int nbatch = (nwave + UB - 1) / UB;
    for (int b = 0; b < nbatch; ++b) {
        if (b > 0)
            issue(b);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int ui = b * UB + u;
            if (ui >= nwave)
                break;
            const int s = wave + kWaves * ui;
            // groups past K read the zero pad
            const int off = 4 * s + g < CPR ? 256 * s + 64 * g : K;
            if constexpr (KERNEL == TWD_KERNEL_DOT) {
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    uint4 x[M];
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        x[m] = *reinterpret_cast<const uint4 *>(smem + m * ldsK + off + 16 * dw);
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
            } else {
                // B operand: this lane's token (column r) over its 64-weight
                // group; B_j word d = activation word 4d + j.
                // Token columns past M read row 0's zero pad.
                const int boff = r < M ? r * ldsK + off : K;
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
    }

    // 4. cross-wave reduction through LDS, then the epilogue
    __syncthreads();  // every wave is done reading activations
    int32_t *red = reinterpret_cast<int32_t *>(smem);  // [wave][m][TW*16]
    constexpr int R = TW * 16;
    if constexpr (KERNEL == TWD_KERNEL_DOT) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                int v = d1[t][m] + (d4[t][m] >> 2) + (d16[t][m] >> 4);
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                if (g == 0)
                    red[(wave * M + m) * R + 16 * t + r] = v;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const v4i c = c0[t] + c3[t] + (c4[t] >> 2) + (c16[t] >> 4);
            if (r < M) {
                int32_t *dst = red + (wave * M + r) * R + 16 * t + 4 * g;
                dst[0] = c.x;
                dst[1] = c.y;
                dst[2] = c.z;
                dst[3] = c.w;
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < M * R; idx += kThreads) {
        const int m = idx / R;
        const int rl = idx - m * R;
        const int n = n0 + rl;
        if (n >= N)
            continue;
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            total += red[(w * M + m) * R + rl] - sq_part[w * M + m];
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if (acc)
            acc[o] = total;
        if (y)
            y[o] = static_cast<float>(total) * xscale[m] * row_gamma(segs, n);
    }
}

constexpr int kMaxKernels = 2 * 3 * 16;  // families x tile counts x widths
constexpr int kMaxLds = 160 * 1024;

using LinearFn = void (*)(const uint4 *, const int8_t *, const float *, int,
                          int, Segments, int32_t *, float *);

template <int KERNEL, int TW, int... Ms>
struct Table {
    static LinearFn get(int M) {
        LinearFn f = nullptr;
        ((M == Ms ? (f = &linear_kernel<KERNEL, Ms, TW>, 0) : 0), ...);
        return f;
    }
    static int lds(int M, int K) {
        int v = 0;
        ((M == Ms ? (v = lds_bytes<Ms, TW>(K), 0) : 0), ...);
        return v;
    }
};

template <int KERNEL, int TW>
using DotTable = Table<KERNEL, TW, 1, 2, 3, 4, 5, 6, 7, 8>;
template <int KERNEL, int TW>
using MfmaTable = Table<KERNEL, TW, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;

LinearFn pick(int kernel, int M, int TW, int K, int *lds) {
    if (kernel == TWD_KERNEL_DOT) {
        switch (TW) {
        case 1: *lds = DotTable<TWD_KERNEL_DOT, 1>::lds(M, K); return DotTable<TWD_KERNEL_DOT, 1>::get(M);
        case 2: *lds = DotTable<TWD_KERNEL_DOT, 2>::lds(M, K); return DotTable<TWD_KERNEL_DOT, 2>::get(M);
        case 4: *lds = DotTable<TWD_KERNEL_DOT, 4>::lds(M, K); return DotTable<TWD_KERNEL_DOT, 4>::get(M);
        }
    } else {
        switch (TW) {
        case 1: *lds = MfmaTable<TWD_KERNEL_MFMA, 1>::lds(M, K); return MfmaTable<TWD_KERNEL_MFMA, 1>::get(M);
        case 2: *lds = MfmaTable<TWD_KERNEL_MFMA, 2>::lds(M, K); return MfmaTable<TWD_KERNEL_MFMA, 2>::get(M);
        case 4: *lds = MfmaTable<TWD_KERNEL_MFMA, 4>::lds(M, K); return MfmaTable<TWD_KERNEL_MFMA, 4>::get(M);
        }
    }
    return nullptr;
}

}  // namespace

// Width dispatch: the VALU dot kernel for narrow widths, matrix cores for
// the wider verification widths; tiles per workgroup grow with N so that
// wide layers still get few, large workgroups.
LinearPlan plan_linear(int M, int K, int N, int forced_kernel) {
    LinearPlan p;
    p.kernel = forced_kernel != TWD_KERNEL_AUTO
                   ? forced_kernel
                   : (M <= 4 ? TWD_KERNEL_DOT : TWD_KERNEL_MFMA);
    const int tiles = (N + 15) / 16;
    p.tiles = 1;
    (void)K;
    p.grid = (tiles + p.tiles - 1) / p.tiles;
    return p;
}

hipError_t launch_linear(const LinearPlan &plan, const uint8_t *w,
                         const int8_t *xq, const float *xscale, int M, int K,
                         int N, const Segments &segs, int32_t *acc, float *y,
                         hipStream_t stream) {
    int lds = 0;
    LinearFn fn = pick(plan.kernel, M, plan.tiles, K, &lds);
    if (!fn)
        return hipErrorInvalidValue;
    if (lds > 65536) {
        // Raise the dynamic-LDS limit to the largest size any call can need,
        // once per kernel (not a stream operation; safe under capture).
        static std::atomic<const void *> raised[kMaxKernels];
        const void *key = reinterpret_cast<const void *>(fn);
        bool done = false;
        int slot = 0;
        for (; slot < kMaxKernels; ++slot) {
            const void *v = raised[slot].load(std::memory_order_acquire);
            if (v == key) {
                done = true;
                break;
            }
            if (v == nullptr)
                break;
        }
        if (!done) {
            hipError_t e = hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kMaxLds);
            if (e != hipSuccess)
                return e;
            if (slot < kMaxKernels) {
                const void *expected = nullptr;
                raised[slot].compare_exchange_strong(expected, key);
            }
        }
    }
    hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(plan.grid)), dim3(kThreads),
                       lds, stream, reinterpret_cast<const uint4 *>(w), xq,
                       xscale, K, N, segs, acc, y);
    return hipGetLastError();
}

}  // namespace twd
