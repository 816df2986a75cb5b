// Streaming-read probe: the rate at which this device reads HBM with 16-byte
// vector loads, the practical ceiling against which the split kernel's
// roofline fraction is read (the published 8 TB/s is a pin rate). The loads
// carry the non-temporal policy (nt) like the split kernels' cache stream; on
// MI355X that reads about 7.0 TB/s against about 6.2 TB/s for plain loads.
// Each workgroup streams one contiguous slice (4 loads in flight per lane)
// and folds it into one float, written only for an impossible sum so the
// loads cannot be removed.
#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

__global__ __launch_bounds__(512) void read_probe_kernel(const float4* __restrict__ p,
                                                         int64_t per_wg, float* out) {
  constexpr int U = 4;
  const float4* base = p + (int64_t)blockIdx.x * per_wg;
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < per_wg; i += (int64_t)blockDim.x * U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      v[u] = j < per_wg ? __builtin_bit_cast(float4, __builtin_nontemporal_load(
                              reinterpret_cast<const u32x4_t*>(base + j)))
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  if (s == -1.0f && threadIdx.x == 0) out[blockIdx.x] = s;
}

sk_status_t read_probe_launch(const void* buf, size_t bytes, int32_t workgroups, float* out,
                              hipStream_t stream) {
  const int64_t per = (int64_t)(bytes / 16) / workgroups;
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(512), 0, stream,
                     reinterpret_cast<const float4*>(buf), per, out);
  return SK_OK;
}

}  // namespace sk
