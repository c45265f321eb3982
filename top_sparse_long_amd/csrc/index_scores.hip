// Lightning-Indexer scoring for the CSA2 hot path on gfx950.
//
//   I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s])      (32 heads x 128 dims)
//
// (CSA2 page, "per-layer attention computation", item 4; DSA page,
// "Lightning Indexer".)  For FP8 rows the kernel follows the dataflow of the
// DSA page's "fp8 and scale absorption" section: the code products are exact
// in fp32, the q scale is folded into the gate, the ReLU-weighted head sum is
// taken, and the per-key scale multiplies the sum.
//
// Decode-shaped work is HBM-bound (132 B of key + 4 B of score per key, 8192
// FLOP), but 58.8 G keys/s at 8 TB/s needs ~480 TFLOP/s, beyond the fp32
// vector units, so the contraction runs on the FP8 MFMA:
//   v_mfma_scale_f32_32x32x64_f8f6f4:  A = q of one query (32 heads x 64 k),
//                                      B = 32 keys (64 k x 32 keys).
// Two MFMAs cover d = 128.  Each lane receives 16 of the 32 heads of one key,
// so the ReLU-weighted head sum is 16 in-register FMAs plus one exchange with
// the lane 32 away.
//
// k-slot assignment: in both operands lane l supplies, for its row/column
// l % 32, the 64 contiguous bytes [64 * (l / 32), +64) of the 128-byte row,
// split as 32 bytes per MFMA.  The two operands use the same assignment, so
// the pair of MFMAs sums every product q[d] * k[d] exactly once whatever the
// hardware's internal k ordering is; only the accumulator layout matters,
// and it is the standard 32x32 one: accumulator j of lane l holds row
// 8 * (j / 4) + 4 * (l / 32) + (j % 4), column l % 32.
#include "kernels.h"

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int IS_WAVES = 4;
constexpr int IS_TILES_PER_WAVE = 16;
constexpr int IS_KEYS_PER_WG = IS_WAVES * 32 * IS_TILES_PER_WAVE;  // 2048

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float load_gate(const IndexScoreArgs& a, int t, int h) {
  if (a.w_bf16) return bf16_to_f32(((const uint16_t*)a.w)[(int64_t)t * a.H + h]);
  return ((const float*)a.w)[(int64_t)t * a.H + h];
}

__device__ __forceinline__ int visible_count(int pos, int ratio) {
  return (int)(((int64_t)pos + 1) / ratio);
}

// Position (within the sequence) scored by column `col` of row t, or -1.
template <bool POOL>
__device__ __forceinline__ int column_position(const IndexScoreArgs& a, int t, int col, int nvis) {
  if (col >= a.n_cols) return -1;
  int p;
  if (POOL) {
    int c = a.cand[(int64_t)t * a.n_cand_blocks + (col >> a.block_shift)];
    if (c < 0) return -1;
    p = (c << a.block_shift) | (col & ((1 << a.block_shift) - 1));
  } else {
    p = col;
  }
  return (p < nvis) ? p : -1;
}

template <bool POOL>
__global__ __launch_bounds__(256) void index_scores_fp8_kernel(IndexScoreArgs a) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int r = lane & 31;

  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int64_t base = a.seq_base[a.q_seq[t]];
  const int col0 = blockIdx.x * IS_KEYS_PER_WG;
  float* out = a.scores + (int64_t)t * a.score_stride;

  // A operand: head r of query t, bytes [64*half, 64*half + 64).
  const uint8_t* qrow = a.q + (int64_t)(t * 32 + r) * a.q_row_stride + 64 * half;
  const v8i A0 = *(const v8i*)(qrow);
  const v8i A1 = *(const v8i*)(qrow + 32);

  // Gates of the 16 heads held by this lane's accumulators, q scale folded in.
  float gate[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int h = 8 * (j >> 2) + 4 * half + (j & 3);
    gate[j] = load_gate(a, t, h) * a.q_scale[(int64_t)(t * 32 + h) * a.q_scale_stride];
  }

  // Dense mode: columns past the visible prefix only need -inf.
  const int limit = POOL ? a.n_cols : min(a.n_cols, nvis);

  for (int it = 0; it < IS_TILES_PER_WAVE; ++it) {
    const int tcol = col0 + (it * IS_WAVES + wave) * 32;
    if (tcol >= a.n_cols) break;
    const int col = tcol + r;
    if (tcol >= limit) {
      if (half == 0 && col < a.n_cols) out[col] = -INFINITY;
      continue;
    }
    const int p = column_position<POOL>(a, t, col, nvis);
    v8i B0 = {0, 0, 0, 0, 0, 0, 0, 0};
    v8i B1 = {0, 0, 0, 0, 0, 0, 0, 0};
    float ks = 0.f;
    if (p >= 0) {
      const uint8_t* krow = a.k + (base + p) * a.k_row_stride + 64 * half;
      B0 = *(const v8i*)(krow);
      B1 = *(const v8i*)(krow + 32);
      ks = a.k_scale[(base + p) * a.k_scale_stride];
    }
    v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A0, B0, acc, 0, 0, 0, 127, 0, 127);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A1, B1, acc, 0, 0, 0, 127, 0, 127);
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) v = fmaf(gate[j], fmaxf(acc[j], 0.f), v);
    v += __shfl_xor(v, 32);
    if (half == 0 && col < a.n_cols) out[col] = (p >= 0) ? v * ks : -INFINITY;
  }
}

// fp32 rows: one thread per column, heads and dims in a plain loop.  Used for
// float inputs (exact for the small-integer configuration).
template <bool POOL>
__global__ __launch_bounds__(256) void index_scores_f32_kernel(IndexScoreArgs a) {
  __shared__ float sq[64 * 128];
  __shared__ float sw[64];
  const int t = blockIdx.y;
  const int H = a.H;
  for (int i = threadIdx.x; i < H * 128; i += 256) {
    const int h = i >> 7, d = i & 127;
    sq[i] = ((const float*)(a.q + (int64_t)(t * H + h) * a.q_row_stride))[d];
  }
  for (int h = threadIdx.x; h < H; h += 256) sw[h] = load_gate(a, t, h);
  __syncthreads();
  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int64_t base = a.seq_base[a.q_seq[t]];
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= a.n_cols) return;
  const int p = column_position<POOL>(a, t, col, nvis);
  float* out = a.scores + (int64_t)t * a.score_stride;
  if (p < 0) {
    out[col] = -INFINITY;
    return;
  }
  const float* krow = (const float*)(a.k + (base + p) * a.k_row_stride);
  float kv[128];
#pragma unroll
  for (int d = 0; d < 128; d += 4) {
    const float4 x = *(const float4*)(krow + d);
    kv[d] = x.x; kv[d + 1] = x.y; kv[d + 2] = x.z; kv[d + 3] = x.w;
  }
  float tot = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < 128; ++d) dot = fmaf(sq[h * 128 + d], kv[d], dot);
    tot = fmaf(sw[h], fmaxf(dot, 0.f), tot);
  }
  out[col] = tot;
}

hipError_t launch_index_scores_fp8(const IndexScoreArgs& a, hipStream_t s) {
  dim3 grid((a.n_cols + IS_KEYS_PER_WG - 1) / IS_KEYS_PER_WG, a.Q);
  if (a.cand)
    hipLaunchKernelGGL(index_scores_fp8_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(index_scores_fp8_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_index_scores_f32(const IndexScoreArgs& a, hipStream_t s) {
  dim3 grid((a.n_cols + 255) / 256, a.Q);
  if (a.cand)
    hipLaunchKernelGGL(index_scores_f32_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(index_scores_f32_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
