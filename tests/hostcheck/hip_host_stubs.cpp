// Host-only stand-ins for the HIP runtime calls and the kernel launchers
// that the planner (fia_api.cpp) references, so that the planner can be built
// with g++ under AddressSanitizer / UndefinedBehaviorSanitizer and driven by
// the phase-1 tests without a GPU.  Every stand-in reports "no device": phase
// 1 never reaches them, and a run on this build fails with FIA_ERR_HIP.
#include <hip/hip_runtime_api.h>

#include "fia.h"
#include "fia_internal.h"

extern "C" {
hipError_t hipGetDevice(int* device) {
  if (device) *device = 0;
  return hipErrorNoDevice;
}
hipError_t hipMalloc(void** ptr, size_t) {
  if (ptr) *ptr = nullptr;
  return hipErrorNoDevice;
}
hipError_t hipFree(void*) { return hipSuccess; }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return hipErrorNoDevice; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNoDevice;
}
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }

// Entry points whose host code lives next to device code (the measured-peak
// probes and the no-allocation run): no device here.
fia_status fia_run_no_alloc(fia_executor*, void*) { return FIA_ERR_HIP; }
fia_status fia_peak_mfma_bf16(int32_t, int32_t, float*, void*) { return FIA_ERR_HIP; }
fia_status fia_peak_hbm_read(const void*, size_t, int32_t, uint32_t*, void*) { return FIA_ERR_HIP; }
}

namespace fia {
hipError_t launch_prefill_bf16(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_bf16(const AttnArgs&, int32_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_merge(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_partition(const AttnArgs&, int32_t*, int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_q8(const AttnArgs&, int32_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fp32(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fill_empty(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sparse(const SparseArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sparse_merge(const SparseArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_read(const AttnArgs&, int32_t, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_gather(const AttnArgs&, int32_t, void*, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_debug_sparse_rows(const SparseArgs&, int32_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
}  // namespace fia
