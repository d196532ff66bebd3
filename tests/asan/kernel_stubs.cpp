// Stand-ins for the kernel launchers of tq_kernels.hip and prefill_kernels.hip, for a CPU-only build of
// tq_host.cpp under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py). Only the host code (codebooks, rotations,
// seeded draws, argument validation) runs in that build; a call that would
// launch a kernel gets an error instead, and every workspace query asks for
// more than any caller passes.
#include <cstddef>
#include <cstdint>

#include "../../kv_cache_vector_turboquant_amd/csrc/tq_internal.h"

namespace tq {
static const size_t kHuge = ~(size_t)0 >> 1;
hipError_t scratch_init(int) { return hipSuccess; }
void *scratch_ptr(int) { return nullptr; }
RecMap cache_map(const tq_kv_cache *, int64_t) { return RecMap(); }
size_t decode_ws_bytes(const tq_ctx *, const tq_kv_cache *, int32_t, int *chunk_out, int *nchunks_out, int) {
  if (chunk_out) *chunk_out = 1024;
  if (nchunks_out) *nchunks_out = 1;
  return kHuge;
}
size_t scores_ws_bytes(const tq_ctx *, int64_t, int64_t, int32_t, int32_t) { return kHuge; }
size_t polar_attention_ws_bytes(const tq_ctx *, const tq_kv_cache *, int32_t) { return kHuge; }
hipError_t launch_quantize_keys(const tq_ctx *, const void *, int, int64_t, int64_t, int64_t, int64_t, const tq_packed *,
                                const RecMap &, float *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quantize_values(const tq_ctx *, const void *, int, int64_t, int64_t, int64_t, int64_t,
                                  const tq_packed *, const RecMap &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_append(const tq_ctx *, const tq_kv_cache *, const void *, const void *, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const tq_ctx *, const tq_kv_cache *, const void *, int, int32_t, float, float *, void *,
                         hipStream_t, const void *, const void *, hipEvent_t, hipEvent_t, int, int, const float *,
                         int64_t, float *) { return hipErrorNotSupported; }
hipError_t launch_read_probe(const void *, size_t, int, uint32_t *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_store(const void *, int, int64_t, int64_t, const float *, int64_t, int64_t, int, float *, int64_t,
                             hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_polar_quantize(const tq_ctx *, const void *, int, int64_t, int64_t, int64_t, const tq_polar_packed *,
                                 int64_t, int64_t, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_polar_scores(const tq_ctx *, const void *, int, int64_t, const tq_polar_packed *, float *, void *,
                               hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_polar_attention(const tq_ctx *, const tq_polar_packed *, const tq_kv_cache *, const void *, int, int32_t,
                                  float, float *, void *, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNotSupported;
}
hipError_t launch_scores(const tq_ctx *, const void *, int, int64_t, const tq_packed *, float *, int32_t, int32_t *,
                         float *, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_merge_partials(const tq_ctx *, const tq_kv_cache *, int32_t, int, float *, int, float *,
                                 hipStream_t) { return hipErrorNotSupported; }
bool prefill_supported(const tq_ctx *, const tq_kv_cache *, int32_t, int) { return false; }
size_t prefill_ws_bytes(const tq_kv_cache *, int32_t, int) { return kHuge; }
hipError_t launch_prefill(const tq_ctx *, const tq_kv_cache *, const void *, int, int32_t, int, int, float, float *,
                          void *, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNotSupported; }
}  // namespace tq
