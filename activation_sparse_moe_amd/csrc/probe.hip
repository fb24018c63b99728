// Streaming-read ceiling of HBM, the reference the layer kernels' achieved
// bandwidth is set against (instrumentation for benchmarks).
//
// A grid-stride sweep of 16-byte non-temporal loads, eight in flight per
// thread.  The XOR of everything read decides one store that practically
// never happens, so the loads cannot be removed and nothing is written.
#include "fff_probe_launch.h"

namespace bffn {
namespace {

constexpr int kProbeInFlight = 8;

__global__ __launch_bounds__(kBlock) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t s) {
  if (blocks <= 0) {
    int64_t resident = 0;
    const hipError_t e = resident_blocks(reinterpret_cast<const void*>(&read_probe_kernel), kBlock, &resident);
    if (e != hipSuccess) return e;
    blocks = (int)resident;
  }
  read_probe_kernel<<<dim3((unsigned)blocks), dim3(kBlock), 0, s>>>(static_cast<const u32x4*>(buf),
                                                                   (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace bffn
