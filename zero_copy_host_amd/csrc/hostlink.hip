// Streaming read / write of pinned host memory by a kernel: the same path (16-byte vector
// loads and stores from mapped host pages) the attention kernels use for the KV cache.
// Its rate is the host-link bound of the layer ("Paper Notes: DirectKV", Motivation and
// Background: the CPU-GPU link, not HBM, limits zero-copy KV access).
#include "dkv_internal.h"

namespace dkv {

// Written only when the xor of the streamed data hits a fixed constant; keeps the loads live.
__device__ uint32_t hostlink_sink;

// Each workgroup reads one contiguous chunk; 8 loads per lane are in flight per step.
__global__ __launch_bounds__(256) void hostlink_read_kernel(const uint4* __restrict__ p, size_t chunk16) {
  const uint4* base = p + (size_t)blockIdx.x * chunk16;
  uint32_t acc = 0;
  size_t i = threadIdx.x;
  const size_t bs = blockDim.x;
  for (; i + 7 * bs < chunk16; i += 8 * bs) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = base[i + u * bs];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < chunk16; i += bs) {
    const uint4 v = base[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) hostlink_sink = acc;
}

__global__ __launch_bounds__(256) void hostlink_write_kernel(uint4* __restrict__ p, size_t chunk16) {
  uint4* base = p + (size_t)blockIdx.x * chunk16;
  const uint4 v = make_uint4(blockIdx.x, threadIdx.x, 0x5A5A5A5Au, 0xA5A5A5A5u);
  for (size_t i = threadIdx.x; i < chunk16; i += blockDim.x) base[i] = v;
}

hipError_t launch_hostlink(void* p, size_t bytes, int mode, int n_wg, hipStream_t s) {
  const size_t chunk16 = bytes / 16 / (size_t)n_wg;
  if (mode == 0) {
    hipLaunchKernelGGL(hostlink_read_kernel, dim3(n_wg), dim3(256), 0, s, reinterpret_cast<const uint4*>(p),
                       chunk16);
  } else {
    hipLaunchKernelGGL(hostlink_write_kernel, dim3(n_wg), dim3(256), 0, s, reinterpret_cast<uint4*>(p), chunk16);
  }
  return hipGetLastError();
}

}  // namespace dkv
