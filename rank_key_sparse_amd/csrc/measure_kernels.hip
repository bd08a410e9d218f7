// Memory-system reference kernels (not part of the decode): a plain copy and
// a plain streaming read over 16-byte granules.  They give the decode's HBM
// figures their reference points: the rate the memory system delivers for a
// pure stream on this part (the practical read ceiling next to the nominal
// peak) and a kernel of known bytes that scales the hardware traffic
// counters.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace loki {

constexpr int kMeasThreads = 256;
constexpr int kMeasUnroll = 8;  // granules per thread per step, all requested before any is used

// Grid-stride copy: step i of a thread moves granules base + u * blockDim
// (u < kMeasUnroll), so one wave's load covers 1 KB contiguous.
__global__ __launch_bounds__(kMeasThreads) void bench_copy_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, size_t n) {
  const size_t span = (size_t)kMeasThreads * kMeasUnroll;
  for (size_t base = (size_t)blockIdx.x * span + threadIdx.x; base < n; base += (size_t)gridDim.x * span) {
    uint4 v[kMeasUnroll];
#pragma unroll
    for (int u = 0; u < kMeasUnroll; ++u) {
      const size_t i = base + (size_t)u * kMeasThreads;
      v[u] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kMeasUnroll; ++u) {
      const size_t i = base + (size_t)u * kMeasThreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Grid-stride read: every granule is folded into a per-thread XOR (so no load
// is dead), reduced over the wave and XORed into *sink once per wave.
__global__ __launch_bounds__(kMeasThreads) void bench_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                  uint32_t* __restrict__ sink) {
  const size_t span = (size_t)kMeasThreads * kMeasUnroll;
  uint32_t acc = 0u;
  for (size_t base = (size_t)blockIdx.x * span + threadIdx.x; base < n; base += (size_t)gridDim.x * span) {
    uint4 v[kMeasUnroll];
#pragma unroll
    for (int u = 0; u < kMeasUnroll; ++u) {
      const size_t i = base + (size_t)u * kMeasThreads;
      v[u] = i < n ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kMeasUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0 && acc) atomicXor(sink, acc);
}

// Enough blocks to fill every CU several times over, each looping.
static unsigned meas_grid(size_t n) {
  const size_t per = (size_t)kMeasThreads * kMeasUnroll;
  const size_t want = (n + per - 1) / per;
  return (unsigned)(want < 8192 ? want : 8192);
}

hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bench_copy_kernel, dim3(meas_grid(n)), dim3(kMeasThreads), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_bench_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bench_read_kernel, dim3(meas_grid(n)), dim3(kMeasThreads), 0, st,
                     static_cast<const uint4*>(src), n, sink);
  return hipGetLastError();
}

}  // namespace loki
