// Machine-peak probes for the roofline denominators: a loop of independent
// bf16 MFMAs (no memory traffic) and a streaming read of a device buffer
// (16-byte non-temporal loads, no reuse).  Their rates, measured on the
// machine that runs the operator, sit beside the published peaks.
#include "fia.h"
#include "fia_device.h"

namespace fia {

// Each wave keeps 8 independent 32x32 accumulators and issues 8 MFMAs per
// iteration: 8 * 32768 flops.  The operands come from the lane index, so
// nothing is loaded; the accumulators' sum is stored so the loop is live.
__global__ __launch_bounds__(256, 2) void peak_mfma_bf16(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t x = 0x3f803f80u ^ (uint32_t)(lane << 3);
  const u32x4 a = {x, x ^ 1u, x ^ 2u, x ^ 3u};
  const u32x4 b = {x ^ 4u, x ^ 5u, x ^ 6u, x ^ 7u};
  f32x16 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = mfma32(a, b, acc[u]);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[u][r];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride read of `bytes` (a multiple of 16) with non-temporal 16-byte
// loads; each thread stores the XOR of what it read.
__global__ __launch_bounds__(256) void peak_hbm_read(const u32x4* buf, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(buf + i);
    const u32x4 v1 = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    acc ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace fia

extern "C" {

fia_status fia_peak_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, void* stream) {
  if (out == nullptr) return FIA_ERR_NULLPTR;
  if (n_workgroups < 1 || iters < 1) return FIA_ERR_PARAM_INVALID;
  fia::peak_mfma_bf16<<<n_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return hipGetLastError() == hipSuccess ? FIA_SUCCESS : FIA_ERR_HIP;
}

fia_status fia_peak_hbm_read(const void* buf, size_t bytes, int32_t n_workgroups, uint32_t* out,
                             void* stream) {
  if (buf == nullptr || out == nullptr) return FIA_ERR_NULLPTR;
  if (n_workgroups < 1 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) {
    return FIA_ERR_PARAM_INVALID;
  }
  fia::peak_hbm_read<<<n_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const fia::u32x4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? FIA_SUCCESS : FIA_ERR_HIP;
}

}  // extern "C"
