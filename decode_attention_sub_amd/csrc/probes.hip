// Bandwidth probes: a streaming read (XOR-reduced so it cannot be elided) that measures the
// practical HBM read ceiling, and a plain copy used to calibrate byte counters.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

constexpr int kProbeGrid = 1024;      // copy probe
constexpr int kProbeBlock = 256;
constexpr int kReadGrid = 8192;       // read probe: 32 workgroups per CU, 8 loads of 16 bytes in
constexpr int kReadUnroll = 8;        // flight per lane, non-temporal (the fastest of a sweep of
                                      // grid, block, unroll and cache policy on MI355X)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeBlock) probe_read_kernel(const uint4* __restrict__ p, size_t n,
                                                                 uint32_t* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load((const u32x4*)(p + i + u * stride));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) { const uint4 a = p[i]; acc ^= a.x ^ a.y ^ a.z ^ a.w; }
  // one word per wave: kReadGrid * 4 words (128 KB) stay inside the documented 1 MB sink
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kProbeBlock / 64) + (threadIdx.x >> 6)] = acc;
}
static_assert(kReadGrid * (kProbeBlock / 64) * 4 <= 4 * 1024 * 256, "read probe sink");

__global__ void __launch_bounds__(kProbeBlock) probe_copy_kernel(const uint4* __restrict__ p,
                                                                 uint4* __restrict__ q, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) q[i] = p[i];
}

}  // namespace

hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, hipStream_t st) {
  probe_read_kernel<<<kReadGrid, kProbeBlock, 0, st>>>((const uint4*)src, bytes / 16, (uint32_t*)sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st) {
  probe_copy_kernel<<<kProbeGrid, kProbeBlock, 0, st>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError();
}

}  // namespace kvq
