// Host-only stand-ins for the device side of libtwd, for the sanitizer build
// of the host code (argument checks, weight format, sweep planner): every
// launch reports hipErrorInvalidValue, and the shape helpers give simple
// answers.  Test infrastructure: the product library never uses this file.
#include "twd_internal.h"

namespace twd {

hipError_t launch_quantize_act(const uint16_t *, int, int, int8_t *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
int narrow_waves(int, int) { return 4; }
bool narrow_supported(int M, int K) { return M >= 1 && M <= 16 && K >= 64; }
hipError_t launch_narrow(const uint8_t *, const void *, bool, const float *, int, int, int,
                         const Segments &, int32_t *, float *, hipStream_t, int) {
    return hipErrorInvalidValue;
}
void rows_shape(int, int, int, int *r, int *w) {
    *r = 4;
    *w = 4;
}
hipError_t launch_rows(const uint8_t *, const void *, bool, const float *, int, int, int,
                       const Segments &, int32_t *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
bool tile_supported(int M, int K) { return M >= 1 && M <= 16 && K <= 3072; }
hipError_t launch_tile(const uint8_t *, const void *, bool, const float *, int, int, int,
                       const Segments &, int32_t *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_staged(int, const uint8_t *, const void *, bool, const float *, int, int, int,
                         const Segments &, int32_t *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
int projection_padded_k(bool, int K) { return K; }
int projection_lds_bytes(bool, int M, int K) { return M * K * 2; }
hipError_t launch_projection(bool, const uint8_t *, const float *, const uint16_t *, int, int,
                             int, float *, uint8_t *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_kv_commit(const KvSegments &, int, int, int, const void *, int,
                            const int32_t *, const int32_t *, const int32_t *, int32_t *,
                            hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_stream_read(const void *, int64_t, uint32_t *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_stream_copy(const void *, void *, int64_t, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_sweep(const twd_sweep_plan &, hipStream_t) { return hipErrorInvalidValue; }
twd_status noalloc_scratch(void *, void **) {
    return set_error(TWD_ERR_HIP, "linear_bf16_noalloc: no device in the host-only build");
}

}  // namespace twd
