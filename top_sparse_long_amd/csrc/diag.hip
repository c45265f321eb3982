// Diagnostic kernels (not on the hot path).
//
// stream_read: the practical HBM read ceiling of the chip, for comparison
// with the hot path's HBM-bound stages.  Every lane reads 16-byte vectors in
// a grid-stride loop, four in flight per iteration, with non-temporal loads
// (the data is streamed once, so it should not displace cached lines); the
// values are summed so the loads are kept, and the sum is stored only if it
// equals a sentinel no real input produces.  On gfx950 this form measured
// about 7.1 TB/s over 2 GiB, against 6.3 TB/s with ordinary loads.
//
// stream_write: fills a buffer with one value through 16-byte non-temporal
// stores in the same grid-stride form -- the write counterpart, and a write
// of known size for calibrating memory-traffic counters.
#include "kernels.h"

namespace csa2 {

typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int SR_THREADS = 256;
constexpr int SR_UNROLL = 4;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const v4f_t* __restrict__ src, size_t n4,
                                                                 float* sink) {
  v4f_t acc = {0.f, 0.f, 0.f, 0.f};
  const size_t step = (size_t)gridDim.x * SR_THREADS * SR_UNROLL;
  for (size_t i = (size_t)blockIdx.x * SR_THREADS * SR_UNROLL + threadIdx.x; i < n4; i += step) {
    v4f_t v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) {
      const size_t j = i + (size_t)u * SR_THREADS;
      v[u] = (j < n4) ? __builtin_nontemporal_load(src + j) : (v4f_t){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc += v[u];
  }
  const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (s == 1234567.f) sink[blockIdx.x] = s;
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(n_blocks), dim3(SR_THREADS), 0, s, (const v4f_t*)src, bytes / 16,
                     sink);
  return hipGetLastError();
}

__global__ __launch_bounds__(SR_THREADS) void stream_write_kernel(v4f_t* __restrict__ dst, size_t n4, float value) {
  const v4f_t v = {value, value, value, value};
  const size_t step = (size_t)gridDim.x * SR_THREADS * SR_UNROLL;
  for (size_t i = (size_t)blockIdx.x * SR_THREADS * SR_UNROLL + threadIdx.x; i < n4; i += step) {
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) {
      const size_t j = i + (size_t)u * SR_THREADS;
      if (j < n4) __builtin_nontemporal_store(v, dst + j);
    }
  }
}

hipError_t launch_stream_write(void* dst, size_t bytes, float value, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(stream_write_kernel, dim3(n_blocks), dim3(SR_THREADS), 0, s, (v4f_t*)dst, bytes / 16, value);
  return hipGetLastError();
}

}  // namespace csa2
