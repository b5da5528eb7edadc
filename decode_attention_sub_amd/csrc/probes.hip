// Bandwidth probes: a streaming read (XOR-reduced so it cannot be elided) that measures the
// practical HBM read ceiling, and a plain copy used to calibrate byte counters.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

constexpr int kProbeGrid = 1024;
constexpr int kProbeBlock = 256;

__global__ void __launch_bounds__(kProbeBlock) probe_read_kernel(const uint4* __restrict__ p, size_t n,
                                                                 uint32_t* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) { const uint4 a = p[i]; acc ^= a.x ^ a.y ^ a.z ^ a.w; }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(kProbeBlock) probe_copy_kernel(const uint4* __restrict__ p,
                                                                 uint4* __restrict__ q, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) q[i] = p[i];
}

}  // namespace

hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, hipStream_t st) {
  probe_read_kernel<<<kProbeGrid, kProbeBlock, 0, st>>>((const uint4*)src, bytes / 16, (uint32_t*)sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st) {
  probe_copy_kernel<<<kProbeGrid, kProbeBlock, 0, st>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError();
}

}  // namespace kvq
