// Measurement probes for the benchmark (not part of the attention path):
// a plain device copy of known size (reference for the HBM byte counters and
// for achievable copy bandwidth), a plain streaming read (achievable read
// bandwidth), and a streaming fill (evicts L2 and the last-level cache
// between timed repetitions).

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(uint4* __restrict__ dst,
                                                             const uint4* __restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming read: each thread keeps eight 16-byte nontemporal loads in
// flight per step (the access pattern the decode's K/V reads aim for).
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4* __restrict__ src, size_t n,
                                                             uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const size_t tile = (size_t)kThreads * U;
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * tile; base < n; base += (size_t)gridDim.x * tile) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const size_t i = base + (size_t)j * kThreads + threadIdx.x;
      v[j] = i < n ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // keeps the loads alive; the condition practically never holds
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void probe_fill_kernel(uint4* __restrict__ dst, size_t n, uint32_t value) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  const uint4 v = make_uint4(value, value, value, value);
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = v;
}

unsigned grid_for(size_t n) {
  const size_t want = (n + kThreads - 1) / kThreads;
  const size_t cap = 256 * 32;  // 32 workgroups per CU on 256 CUs
  return (unsigned)(want < cap ? (want ? want : 1) : cap);
}

}  // namespace

#define PROBE_API __attribute__((visibility("default")))

extern "C" {

// bytes must be a multiple of 16; pointers 16-byte aligned device pointers.
PROBE_API int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16) return -1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(grid_for(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

PROBE_API int pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16) return -1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid_for(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), n, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

PROBE_API int pkv_probe_fill(void* dst, size_t bytes, uint32_t value, void* stream) {
  if (!dst || bytes % 16) return -1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(probe_fill_kernel, dim3(grid_for(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), n, value);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
