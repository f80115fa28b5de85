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

// Streaming read of `bytes` (a multiple of 16): workgroups take contiguous
// 32 KiB blocks in turn, each thread 8 non-temporal 16-byte loads in flight
// (a wave reads 1 KiB runs), then the tail past the last whole block; each
// thread stores the XOR of what it read.
__global__ __launch_bounds__(256) void peak_hbm_read(const u32x4* buf, int64_t n16, uint32_t* out) {
  constexpr int BLK = 8 * 256;   // 16-byte units per block
  const int64_t n_blk = n16 / BLK;
  uint32_t acc = 0;
  for (int64_t blk = blockIdx.x; blk < n_blk; blk += gridDim.x) {
    const u32x4* p = buf + blk * BLK + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int64_t i = n_blk * BLK + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
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
