// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// that the library's host side (aq_api.cpp, aq_plan.cpp) makes, so that the
// host side builds with a plain C++ compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer and runs without a GPU.  Every launcher returns
// g_forced, which the check program sets to force a launch failure
// (hipErrorLaunchFailure) or success, and counts its calls.
#include <hip/hip_runtime_api.h>

#include "../../mixed_precision_int_amd/csrc/aq_internal.h"

hipError_t g_forced = hipSuccess;
int g_launches = 0;

namespace {
hipError_t launched() {
  ++g_launches;
  return g_forced;
}
}  // namespace

namespace aq {
hipError_t launch_pack(const float *, const aq_packed &, hipStream_t, bool) { return launched(); }
hipError_t launch_quant_act(const float *, int, int, int8_t *, float *, hipStream_t) { return launched(); }
hipError_t launch_decode(const PackedView &, const int8_t *, const float *, int, const float *, float *, int,
                         void *, int32_t *, hipStream_t, bool) {
  return launched();
}
hipError_t launch_quant_act_grouped(const float *, int, int, int8_t *, float *, hipStream_t) { return launched(); }
hipError_t launch_prefill(const PackedView &, const int8_t *, const float *, int, const float *, float *,
                          int32_t *, hipStream_t, const int8_t *, const aq_transform_tables *) {
  return launched();
}
hipError_t launch_prefill_dense(const int8_t *, const float *, int, int, int, const int8_t *, const float *, int,
                                const float *, float *, int32_t *, hipStream_t, const int8_t *,
                                const aq_transform_tables *) {
  return launched();
}
hipError_t launch_prefill_dense_grouped(const int8_t *, const float *, int, int, const int8_t *, const float *, int,
                                        const float *, float *, int32_t *, hipStream_t) {
  return launched();
}
hipError_t launch_prefill_big(const int8_t *, const float *, int, int, const int8_t *, const float *, int,
                              const float *, float *, int32_t *, hipStream_t, const int8_t *,
                              const aq_transform_tables *) {
  return launched();
}
hipError_t launch_expand(const PackedView &w, void *ws, hipStream_t, const int8_t **E, const float **Es) {
  expand_layout(w, ws, E, Es);
  return launched();
}
void expand_layout(const PackedView &w, const void *ws, const int8_t **E, const float **Es) {
  const int8_t *e = static_cast<const int8_t *>(ws);
  *E = e;
  *Es = reinterpret_cast<const float *>(e + (((size_t)w.N * w.K + 255) & ~(size_t)255));
}
hipError_t launch_transform(int, const float *, float *, int, int, const int8_t *, const int8_t *, const float *,
                            const TransformTables &, hipStream_t) {
  return launched();
}
hipError_t launch_quant_act_transformed(const float *, int, int, const int8_t *, const TransformTables &,
                                        int8_t *, float *, hipStream_t) {
  return launched();
}
hipError_t launch_decode_transformed(const PackedView &, const int8_t *, const float *, int, const float *,
                                     float *, int, void *, const int8_t *, const TransformTables &,
                                     hipStream_t) {
  return launched();
}
hipError_t launch_decode_fp32(const PackedView &, const float *, int, const float *, float *, int, void *,
                              hipStream_t) {
  return launched();
}
hipError_t launch_zero_counters(void *, hipStream_t) { return launched(); }
hipError_t decode_scratch(hipStream_t, void **out) {
  static unsigned char fake[64];
  *out = fake;
  return launched();
}
}  // namespace aq

// The HIP runtime calls of the host side, without a runtime: the copies of
// aq_pack_weights fail when a launch failure is forced; one device of 256
// compute units.
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) { return g_forced; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
