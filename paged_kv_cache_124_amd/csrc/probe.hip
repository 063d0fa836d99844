// Measurement helper: the achievable HBM read rate of this GPU, against which
// the decode kernels' rates are read (the decode path is a bandwidth-bound
// gather: "PagedAttention: Virtual Memory for the KV Cache", section 13).
// A plain streaming read -- every byte of a buffer once, in 4 KiB pieces of
// 16-byte loads, no LDS, no compute beyond an XOR that keeps the loads alive --
// is the ceiling a kernel that streams whole blocks can approach.  The loads
// take either the default cache policy or the non-temporal one (the "nt"
// modifier: lines not kept for reuse), which the decode kernels use for the KV.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_probe.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

// Wave w reads the 4 KiB pieces w, w + W, w + 2W, ... of the buffer (W waves
// in the launch), four pieces (16 loads of 16 bytes per lane) in flight; the
// 64 lanes of one load cover 1 KiB contiguous, as the decode's block copies do.
template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ buf, int64_t pieces,
                                                         uint32_t* __restrict__ sink) {
  constexpr int UNR = 4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t W = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (int64_t b = wave; b < pieces; b += W * UNR) {
    uint4 v[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t bb = b + u * W < pieces ? b + u * W : b;  // past the end: read piece b again (counted once below)
      const uint4* p = buf + bb * 256;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[u][k] = load16<NT>(p + k * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[u][k].x ^ v[u][k].y ^ v[u][k].z ^ v[u][k].w;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) acc ^= __shfl_xor(acc, sh);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;  // wave 0's XOR: one word per workgroup
}

}  // namespace
}  // namespace pa

extern "C" int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, int nontemporal,
                             void* stream) {
  using namespace pa;
  if (bytes % 4096 != 0 || workgroups < 1 || workgroups > 65535) return 1;
  if (bytes == 0) return 0;
  if (!buf || !sink) return 1;
  if (nontemporal != 0 && nontemporal != 1) return 1;
  const auto kernel = nontemporal ? read_probe_kernel<true> : read_probe_kernel<false>;
  kernel<<<dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), static_cast<int64_t>(bytes / 4096), sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}
