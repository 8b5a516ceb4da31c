// probe.hip -- a streaming-read probe: the HBM read rate a plain kernel reaches on this GPU,
// the ceiling the attention kernels' byte rates are read against (include/kvq_probe.h).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup w reads the w-th of `grid` equal contiguous slices with non-temporal 16-byte
// loads, kUnroll per thread at a time, and folds them by XOR into one word per workgroup
// (written, so no load is dead).  n16 = number of 16-byte units, a multiple of the grid's
// units per round so every load is in bounds.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4 *buf, size_t n16, uint32_t *sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const size_t per = n16 / gridDim.x;
  const uint4 *p = buf + per * blockIdx.x;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i + (kUnroll - 1) * kThreads < per; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + i + k * kThreads));
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kThreads; ++i) t ^= red[i];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" int kvq_hbm_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *sink, void *stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) || workgroups < 1) return -1;
  const size_t round = static_cast<size_t>(workgroups) * kThreads * kUnroll * 16;
  if (bytes < round || bytes % round != 0) return -1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
