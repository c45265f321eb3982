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
//
// mfma_valu: whether matrix-core products and vector ALU work on the same
// SIMD overlap.  256 workgroups of eight waves (two per SIMD, the occupancy
// of the hot path's MFMA kernels) each run a loop of eight independent
// v_mfma_f32_32x32x16_f16 products, 64 independent fp32 FMAs, or both; the
// caller times the three launches.  If the two kinds of work overlapped,
// both would take about as long as the longer one alone.
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

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
constexpr int MV_THREADS = 512;

template <bool MF, bool VA>
__global__ __launch_bounds__(MV_THREADS) void mfma_valu_kernel(int iters, float* sink) {
  const float seed = (float)(threadIdx.x & 31) * 0.001f;
  v8h_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = (_Float16)(seed * (float)(e + i + 1));
      b[i][e] = (_Float16)(seed * (float)(3 * e + i + 1));
    }
  v16f_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (v16f_t){};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(i + 1);
  const float gm = 1.0f - seed;
  for (int it = 0; it < iters; ++it) {
    if (MF) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m & 1], b[m & 1], acc[m & 3], 0, 0, 0);
    }
    if (VA) {
#pragma unroll
      for (int v = 0; v < 64; ++v) x[v & 15] = fmaf(x[v & 15], gm, seed);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  sink[blockIdx.x * MV_THREADS + threadIdx.x] = s;
}

hipError_t launch_mfma_valu(int mode, int iters, float* sink, hipStream_t s) {
  const dim3 grid(MV_BLOCKS), block(MV_THREADS);
  if (mode == 1) hipLaunchKernelGGL((mfma_valu_kernel<true, false>), grid, block, 0, s, iters, sink);
  else if (mode == 2) hipLaunchKernelGGL((mfma_valu_kernel<false, true>), grid, block, 0, s, iters, sink);
  else hipLaunchKernelGGL((mfma_valu_kernel<true, true>), grid, block, 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace csa2
