// Straight-line matrix-core kernel of the W2A8 ternary linear, gfx950: one
// pass over the weights with every load issued up front, for drafted blocks
// (M = 2..16) whose activation slices fit in registers.
//
// What they compute (BitMTP page, ai.info AI summary): ternary BitNet b1.58
// weights ("What This Paper Is About"), 8-bit activations ("Main Findings":
// W2A8), and the packed low-bit operator M1 picks by replay width
// ("Methodology in Plain English", paragraph 3):
// acc[m][n] = sum_k q[m][k] t[n][k] in int32, y = acc * s_m * gamma(n).
// With FUSED the per-token absmax int8 quantization of the bf16 activations
// (same arithmetic as the stand-alone quantizer) happens inside.
//
// Work split.  A workgroup of NW = 4, 8 or 16 waves owns 16 weight rows and
// all of K.  Wave w takes the 256-wide K slices w, w + NW, ..., exactly U of
// them (U is a
// compile-time count, so every load is straight-line code; a wave with one
// slice fewer loads a slice whose activations are zero).  All loads are
// buffer loads: 32-bit offsets against a descriptor whose size bound makes
// out-of-range reads return zero, so rows past N and activations past K need
// no clamping.  They are issued in order -- this wave's activation slices
// first, then its weights -- so the wave waits for the activations alone
// before staging them, and for each weight slice only when it is consumed:
// quantization and decode overlap the weight stream.
//
// In one slice, lane l loads 16 bytes (64 weights) of row l % 16 at K offset
// 256 s + 64 (l / 16); the wave covers 16 rows x 256 weights.  Each wave
// stages the int8 activations of its own slices in a private LDS region, so
// the only cross-wave synchronization is the row absmax (FUSED) and the
// final sum.
//
// Decode.  A 32-bit word holds 16 codes c = t + 1; masking with 0x03030303,
// 0x0C0C0C0C, 0x30303030 gives byte planes holding c, 4c, 16c for elements
// 4j..4j+3 (j = 0, 1, 2) and (w >> 6) & 0x03030303 gives plane 3.  Plane j of
// the lane's four words is the A operand of a 16x16x64 int8 MFMA (row =
// lane % 16, K group = lane / 16); the tokens fill the B columns, a zero
// block beyond M.  The planes scaled by 4 and 16 have their own
// accumulators, shifted back exactly at the end; sum q t = sum q c - sum q.
// The staged activations are stored permuted within each 16-word group so
// that one 16-byte LDS read yields a B operand.
#include "kernel_common.h"

namespace twd {
namespace {

using namespace kern;

// Buffer resource word 3 for raw (untyped) loads on CDNA: 32-bit data format.
constexpr int kRawBufferFlags = 0x00020000;
// An offset past every buffer bound: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Per-wave LDS region: M staged rows of U slices, then a zero block.  The
// row stride is padded by 16 bytes so that the 16 token rows a B-operand read
// touches fall on 16 different 4-bank groups (64 banks of 4 bytes).
template <int U>
__host__ __device__ constexpr int row_stride() { return U * 256 + 16; }

template <int M, int U>
__host__ __device__ constexpr int wave_bytes() { return M * row_stride<U>() + 64; }

// LDS: per-wave regions | partials [M][17][wave] (16 rows, padded so that
// the 16 token columns a write touches fall on different banks) | absmax
// partials [wave, DPP row][M] | row-sum partials [wave, DPP row][M].
constexpr int kRedStride = 17;

template <int M, int NW, int U>
__host__ __device__ constexpr int lds_bytes() {
    return NW * wave_bytes<M, U>() + M * kRedStride * NW * 4 + 2 * 4 * NW * M * 4;
}

// Where lane l's activation word (elements 4l..4l+3 of the slice) is staged:
// word 16g + 4d + j goes to 16g + 4j + d, so the four words of plane j of K
// group g are contiguous.
__device__ __forceinline__ int staged_word(int lane) {
    return (lane & 48) | ((lane & 3) << 2) | ((lane >> 2) & 3);
}

template <int M, int NW, int U, bool FUSED>
__global__ __launch_bounds__(64 * NW) void mfma_kernel(
    const uint8_t *__restrict__ W, const void *__restrict__ act,
    const float *__restrict__ xscale, int32_t *__restrict__ acc, float *__restrict__ y, int K,
    int N, Segments segs) {
    constexpr int P = NW;  // partial sums per output
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int row_bytes = K >> 2;

    uint8_t *own = smem + wave * wave_bytes<M, U>();
    int32_t *red = reinterpret_cast<int32_t *>(smem + NW * wave_bytes<M, U>());
    uint32_t *st_max = reinterpret_cast<uint32_t *>(red + M * kRedStride * P);  // [4 NW][M]
    int32_t *st_sum = reinterpret_cast<int32_t *>(st_max + 4 * NW * M);  // [4 NW][M]
    const int part = wave * 4 + (lane >> 4);  // this lane's DPP row in the workgroup

    // 1. activation loads: lane l takes elements 256 s + 4 l .. + 3 of each
    //    row for this wave's slices s = wave + NW u (zeros past K)
    constexpr int kEl = FUSED ? 2 : 1;  // bytes per element
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(act), 0, M * K * kEl, kRawBufferFlags);
    uint2 xb[FUSED ? M : 1][U];
    uint32_t xi[FUSED ? 1 : M][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k0 = 256 * (wave + NW * u) + 4 * lane;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint32_t off =
                k0 < K ? static_cast<uint32_t>((m * K + k0) * kEl) : kOutOfRange;
            if constexpr (FUSED) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0);
                xb[m][u] = make_uint2(v[0], v[1]);
            } else {
                xi[m][u] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
            }
        }
    }

    // 2. weight loads against this workgroup's 16 rows; rows past N fall
    //    outside the descriptor (zeros, never stored), K groups past the
    //    row end read the next row (their activations are zero)
    const int rows = min(16, N - n0);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(W + static_cast<int64_t>(n0) * row_bytes), 0,
        rows * row_bytes, kRawBufferFlags);
    const uint32_t wbase = static_cast<uint32_t>(r * row_bytes + 16 * g);
    uint4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(
            wr, wbase + 64u * static_cast<uint32_t>(wave + NW * u), 0, kWeightPolicy);
        a[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    // keep every load issued before any use (the scheduler would otherwise
    // hoist activation math, and its wait, above the weight loads)
    __builtin_amdgcn_sched_barrier(0);
    // the segment scale of this thread's output (step 5) and the output
    // pointers: their kernel-argument loads wait here, in the shadow of the
    // activation loads
    const int n_o = n0 + (tid & 15);
    float gam_o = row_gamma(segs, n_o);
    settle_v(gam_o);
    settle_s(acc);
    settle_s(y);
    __builtin_amdgcn_sched_barrier(0);

    // 3. own activation slices -> LDS as int8, with this wave's row sums;
    //    the dequantization factors of this thread's output (step 5) are
    //    settled here, in the shadow of the weight loads
    const int slot = 4 * staged_word(lane);
    float scale_o = 0.0f;
    if constexpr (!FUSED)
        scale_o = xscale[min(tid >> 4, M - 1)];
    int sq[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        sq[m] = 0;
    if constexpr (FUSED) {
        // row absmax: per-lane partials, reduced over each DPP row for all
        // rows at once, 16 partials per row to LDS
        uint32_t amv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u16x2 am2 = {0, 0};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                am2 = absmax_pair(am2, xb[m][u].x);
                am2 = absmax_pair(am2, xb[m][u].y);
            }
            amv[m] = absmax_bits(am2);
        }
        row_max16<M>(amv);
        if ((lane & 15) == 15) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                st_max[part * M + m] = amv[m];
        }
        __syncthreads();  // row absmax partials (LDS only)
        // lane m combines row m and divides once for it (correctly rounded
        // fp32 division, build flag, as in the stand-alone quantizer; an
        // all-zero row quantizes to zeros)
        uint32_t am_l = 0;
        if (lane < M) {
#pragma unroll
            for (int i = 0; i < 4 * NW; ++i)
                am_l = max(am_l, st_max[i * M + lane]);
        }
        const float a_l = __uint_as_float(am_l);
        const float inv_l = a_l > 0.0f ? 127.0f / a_l : 0.0f;
        // the scale of this thread's output row (step 5), from lane
        // tid / 16 of this wave, which holds that row's absmax
        const float a_o = __int_as_float(
            __builtin_amdgcn_ds_bpermute(4 * ((tid >> 4) & 15), __float_as_int(a_l)));
        scale_o = a_o / 127.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), m));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t q = quant4(xb[m][u].x, xb[m][u].y, inv);
                *reinterpret_cast<uint32_t *>(own + m * row_stride<U>() + u * 256 + slot) = q;
                sq[m] = sdot4(q, kOnes, sq[m]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                *reinterpret_cast<uint32_t *>(own + m * row_stride<U>() + u * 256 + slot) = xi[m][u];
                sq[m] = sdot4(xi[m][u], kOnes, sq[m]);
            }
    }
    if (lane < 4)  // zero block behind the token columns past M
        *reinterpret_cast<uint4 *>(own + M * row_stride<U>() + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
    row_sum16<M>(sq);
    if ((lane & 15) == 15) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            st_sum[part * M + m] = sq[m];
    }
    settle_v(scale_o);
    __builtin_amdgcn_sched_barrier(0);
    // the wave reads back only its own LDS region: its writes are ordered
    // before its reads, no workgroup barrier needed
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 4. decode + multiply-accumulate, one slice at a time as it arrives
    {
        v4i c0 = {0, 0, 0, 0}, c3 = c0, c4 = c0, c16 = c0;
        // B operand of plane j: token r's K group g; columns past M read
        // the zero block
        const uint8_t *bsrc = r < M ? own + r * row_stride<U>() + 64 * g : own + M * row_stride<U>();
        const int ustep = r < M ? 256 : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint8_t *bu = bsrc + u * ustep;
            const v4i b0 = *reinterpret_cast<const v4i *>(bu);
            const v4i b1 = *reinterpret_cast<const v4i *>(bu + 16);
            const v4i b2 = *reinterpret_cast<const v4i *>(bu + 32);
            const v4i b3 = *reinterpret_cast<const v4i *>(bu + 48);
            const v4i w = {static_cast<int>(a[u].x), static_cast<int>(a[u].y),
                           static_cast<int>(a[u].z), static_cast<int>(a[u].w)};
            const v4i p0 = w & static_cast<int>(kPlane0);
            const v4i p1 = w & static_cast<int>(kPlane1);
            const v4i p2 = w & static_cast<int>(kPlane2);
            const v4i p3 = (w >> 6) & static_cast<int>(kPlane0);
            c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p0, b0, c0, 0, 0, 0);
            c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p1, b1, c4, 0, 0, 0);
            c16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p2, b2, c16, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(p3, b3, c3, 0, 0, 0);
        }
        // lane (r, g) holds rows 4g .. 4g+3 of token r: partials [M][16][wave],
        // each less the row sum of q over this wave's slices
        if (r < M) {
            int qw = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qw += st_sum[(wave * 4 + i) * M + r];
            const v4i c = c0 + c3 + (c4 >> 2) + (c16 >> 4) - qw;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[(r * kRedStride + 4 * g + i) * P + wave] = c[i];
        }
    }

    // 5. one thread per output (M * 16 <= 256 <= 64 NW) adds its partials,
    //    takes off the row sum and dequantizes
    __syncthreads();
    if (tid < M * 16 && n_o < N) {
        const int m = tid >> 4;
        int total = 0;
#pragma unroll
        for (int p = 0; p < P; p += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(red + (m * kRedStride + (tid & 15)) * P + p);
            total += v.x + v.y + v.z + v.w;
        }
        const int64_t o = static_cast<int64_t>(m) * N + n_o;
        if (acc)
            acc[o] = total;
        if (y)
            y[o] = static_cast<float>(total) * scale_o * gam_o;
    }
}

using Fn = void (*)(const uint8_t *, const void *, const float *, int32_t *, float *, int, int,
                    Segments);

template <int M, int NW, bool FUSED, int... Us>
bool pick_u(int U, Fn *fn, int *lds) {
    bool found = false;
    auto take = [&](auto uc) {
        constexpr int Uc = decltype(uc)::value;
        if constexpr (narrow_fits(M, Uc)) {
            static_assert(lds_bytes<M, NW, Uc>() <= 160 * 1024, "LDS budget");
            *fn = &mfma_kernel<M, NW, Uc, FUSED>;
            *lds = lds_bytes<M, NW, Uc>();
            found = true;
        }
    };
    ((U == Us ? (take(std::integral_constant<int, Us>{}), 0) : 0), ...);
    return found;
}

// U = ceil(ceil(K / 256) / NW) <= 8, 4, 2 for NW = 4, 8, 16 (K <= 8192)
template <bool FUSED, int... Ms>
bool pick_m(int M, int NW, int U, Fn *fn, int *lds) {
    bool found = false;
    if (NW == 4)
        ((M == Ms ? (found = pick_u<Ms, 4, FUSED, 1, 2, 3, 4, 5, 6, 7, 8>(U, fn, lds)) : false), ...);
    else if (NW == 8)
        ((M == Ms ? (found = pick_u<Ms, 8, FUSED, 1, 2, 3, 4>(U, fn, lds)) : false), ...);
    else if (NW == 16)
        ((M == Ms ? (found = pick_u<Ms, 16, FUSED, 1, 2>(U, fn, lds)) : false), ...);
    return found;
}

}  // namespace

// Waves per 16-row workgroup: the fewest of 4, 8, 16 whose K share per wave
// (U slices) keeps M x U activation words per lane within the register
// budget -- more waves split K finer, for wide M or long K.
int narrow_waves(int M, int K) {
    const int S = (K + 255) / 256;
    for (int nw = 4; nw <= 16; nw *= 2)
        if (narrow_fits(M, (S + nw - 1) / nw))
            return nw;
    return 0;
}

bool narrow_supported(int M, int K) {
    return M >= 1 && M <= TWD_MAX_M && K >= 1 && narrow_waves(M, K) != 0;
}

hipError_t launch_narrow(const uint8_t *w, const void *act, bool fused,
                         const float *xscale, int M, int K, int N,
                         const Segments &segs, int32_t *acc, float *y,
                         hipStream_t stream, int waves) {
    const int NW = waves ? waves : narrow_waves(M, K);
    if (NW != 4 && NW != 8 && NW != 16)
        return hipErrorInvalidValue;
    const int S = (K + 255) / 256;
    const int U = (S + NW - 1) / NW;  // 256-wide slices per wave
    Fn fn = nullptr;
    int lds = 0;
    const bool ok =
        fused ? pick_m<true, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(M, NW, U, &fn, &lds)
              : pick_m<false, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(M, NW, U, &fn, &lds);
    if (!ok)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, dim3((N + 15) / 16), dim3(64 * NW), lds, stream, w, act,
                       xscale, acc, y, K, N, segs);
    return hipGetLastError();
}

}  // namespace twd
