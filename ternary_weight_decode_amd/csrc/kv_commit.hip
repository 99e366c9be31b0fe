// Accepted-prefix KV commit over geometrically sized shared segments
// (BitMTP page, ai.info AI summary, "Methodology in Plain English",
// paragraph 3: the state triple of committed prefix, materialized causal KV
// length and pending suffix, kept consistent by a length identity; one
// physical KV buffer per segment, shared by every captured graph, with
// capacities growing geometrically; "Key Contributions", item 1: graphs
// reuse the shared history instead of copying it).
//
// State (device int32[4]): P committed, L materialized, S pending, error.
// Identity P == L + S.  Segment s holds C0 2^s positions after segments
// 0..s-1, so position p is in segment s = bitlength(p / C0 + 1) - 1 (integer
// division) at offset p - C0 (2^s - 1); its buffer is [layer][K, V][C0 2^s]
// [row].  A commit stores the first n_mat rows of the block a pass computed
// for positions L.. and moves the state to (P + n_new, L + n_mat, P - L +
// n_new - n_mat); the counts live in device memory, so a captured graph
// replays commits whose sizes are only known on the device.
//
// Every workgroup reads the same inputs and so takes the same decision; one
// thread writes the new state to a separate output (the caller alternates
// two state words), so no workgroup can see a half-updated state.
#include "twd_internal.h"

namespace twd {
namespace {

constexpr int kKvThreads = 256;

__global__ __launch_bounds__(kKvThreads) void kv_commit_kernel(
    const uint4 *__restrict__ block, const int32_t *__restrict__ n_mat_p,
    const int32_t *__restrict__ n_new_p, const int32_t *__restrict__ state_in,
    int32_t *__restrict__ state_out, int C0, int row16, int W, KvSegments segs) {
    const int j = blockIdx.x;       // block row
    const int lk = blockIdx.y;      // layer * 2 + (K, V)
    const int P = state_in[0], L = state_in[1], S = state_in[2], err = state_in[3];
    const int n_mat = *n_mat_p, n_new = *n_new_p;
    int e = err;
    if (e == 0 && (L < 0 || S < 0 || P != L + S))
        e = 1;
    if (e == 0 && (n_mat < 0 || n_mat > W || n_new < 0 ||
                   static_cast<int64_t>(P) + n_new > 0x7FFFFFFF ||
                   static_cast<int64_t>(L) + n_mat > static_cast<int64_t>(P) + n_new))
        e = 2;
    if (e == 0 && static_cast<int64_t>(L) + n_mat > segs.capacity)
        e = 3;
    if (j == 0 && lk == 0 && threadIdx.x == 0) {
        if (e == 0) {
            state_out[0] = P + n_new;
            state_out[1] = L + n_mat;
            state_out[2] = P + n_new - (L + n_mat);
            state_out[3] = 0;
        } else {
            state_out[0] = P;
            state_out[1] = L;
            state_out[2] = S;
            state_out[3] = e;
        }
    }
    if (e != 0 || j >= n_mat)
        return;
    const int p = L + j;
    const uint32_t q = static_cast<uint32_t>(p / C0 + 1);
    const int s = 31 - __builtin_clz(q);
    const int64_t cap = static_cast<int64_t>(C0) << s;
    const int64_t off = p - (cap - C0);  // C0 (2^s - 1) positions before segment s
    const uint4 *src = block + (static_cast<int64_t>(lk) * W + j) * row16;
    uint4 *dst = static_cast<uint4 *>(segs.ptr[s]) + (lk * cap + off) * row16;
    for (int i = threadIdx.x; i < row16; i += kKvThreads)
        dst[i] = src[i];
}

}  // namespace

hipError_t launch_kv_commit(const KvSegments &segs, int C0, int layers, int row_bytes,
                            const void *block, int W, const int32_t *n_mat,
                            const int32_t *n_new, const int32_t *state_in, int32_t *state_out,
                            hipStream_t stream) {
    hipLaunchKernelGGL(kv_commit_kernel, dim3(W, 2 * layers), dim3(kKvThreads), 0, stream,
                       static_cast<const uint4 *>(block), n_mat, n_new, state_in, state_out, C0,
                       row_bytes / 16, W, segs);
    return hipGetLastError();
}

}  // namespace twd
