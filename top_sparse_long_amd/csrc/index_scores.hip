// Lightning-Indexer scoring for the CSA2 hot path on gfx950.
//
//   I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s])      (32 heads x 128 dims)
//
// (CSA2 page, "per-layer attention computation", item 4; DSA page,
// "Lightning Indexer".)  For FP8 rows the kernel follows the dataflow of the
// DSA page's "fp8 and scale absorption" section: the code products are exact,
// the q scale is folded into the gate, the ReLU-weighted head sum is taken,
// and the per-key scale multiplies the sum.
//
// Contraction: every E4M3 code is exactly representable in f16, so the codes
// are widened in registers (v_cvt_scalef32_pk_f16_fp8 with scale 1) and fed to
// v_mfma_f32_32x32x16_f16, whose 22-bit products are exact and whose sums
// carry fp32 precision.  The FP8 MFMA forms of gfx950 were measured to
// accumulate with about 17 significant bits, which on Gaussian data with the
// usual cancellation breaks a 1e-3 relative bound on the scores; the f16 form
// keeps the decode kernel HBM-bound all the same (8 f16 MFMAs of 32 cycles
// per 4 KB key tile per wave).
//
// Layout: A = q of one query (32 heads x 16 k), B = 32 keys (16 k x 32 keys);
// eight MFMAs cover d = 128.  Lane l owns row/column l % 32 and the 64
// contiguous bytes [64 * (l / 32), +64) of that 128-byte row (8 bytes per
// MFMA); both operands use the same assignment, so every product q[d] k[d]
// is summed exactly once.  The accumulator layout is the standard 32x32 one
// (accumulator j of lane l: head 8 (j / 4) + 4 (l / 32) + j % 4, key l % 32),
// so the ReLU-weighted head sum is 16 in-register FMAs plus one exchange with
// the lane 32 away.  Each wave loads all of its tiles before computing, so
// about 16 KB per wave are in flight.
//
// Optional fused output: the block maximum of every block_size (<= 32)
// consecutive columns (the first step of the CSA2 page's candidate pool:
// "blocks are not compression"), taken over the scores in registers.
#include "kernels.h"

namespace csa2 {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

#ifndef CSA2_IS_WAVES
#define CSA2_IS_WAVES 4
#endif
#ifndef CSA2_IS_TILES
#define CSA2_IS_TILES 4
#endif
constexpr int IS_WAVES = CSA2_IS_WAVES;                      // waves per workgroup
constexpr int IS_TILES = CSA2_IS_TILES;                      // 32-key tiles per wave
constexpr int IS_KEYS_PER_WG = IS_WAVES * 32 * IS_TILES;      // 512

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
    const int c = a.cand[(int64_t)t * a.n_cand_blocks + (col >> a.block_shift)];
    if (c < 0) return -1;
    p = (c << a.block_shift) | (col & ((1 << a.block_shift) - 1));
  } else {
    p = col;
  }
  return (p < nvis) ? p : -1;
}

// 8 E4M3 codes (two dwords) -> 8 f16 values, exactly.
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool POOL, bool W_BF16>
__global__ __launch_bounds__(64 * IS_WAVES) void index_scores_fp8_kernel(IndexScoreArgs a) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int r = lane & 31;

  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int64_t base = a.seq_base[a.q_seq[t]];
  const int col0 = blockIdx.x * IS_KEYS_PER_WG;
  float* out = a.scores + (int64_t)t * a.score_stride;
  // Dense mode: columns past the visible prefix only need -inf.
  const int limit = (nvis <= 0) ? 0 : (POOL ? a.n_cols : min(a.n_cols, nvis));

  // q (head r, bytes [64 half, +64)) and the gate of head r are loaded
  // first and used after the key loads are issued, so one round trip covers
  // all of them.
  v4u qraw[4];
  {
    const v4u* qsrc = (const v4u*)(a.q + (int64_t)(t * 32 + r) * a.q_row_stride + 64 * half);
#pragma unroll
    for (int j = 0; j < 4; ++j) qraw[j] = qsrc[j];
  }
  float g_r;
  if (W_BF16)
    g_r = bf16_to_f32(((const uint16_t*)a.w)[(int64_t)t * 32 + r]);
  else
    g_r = ((const float*)a.w)[(int64_t)t * 32 + r];
  const float qs_r = a.q_scale[(int64_t)(t * 32 + r) * a.q_scale_stride];

  if (limit == 0) {
    // nothing visible: every column of this workgroup is -inf
    for (int c = col0 + threadIdx.x; c < min(a.n_cols, col0 + IS_KEYS_PER_WG); c += 64 * IS_WAVES) {
      out[c] = -INFINITY;
      if (!POOL && a.block_max && (c & ((1 << a.block_shift) - 1)) == 0)
        a.block_max[(int64_t)t * a.block_max_stride + (c >> a.block_shift)] = -INFINITY;
    }
    return;
  }

  // This wave's tiles: columns col0 + (i * IS_WAVES + wave) * 32 + [0, 32).
  // Every load is unconditional: lanes whose column scores nothing read
  // position 0 of the sequence (visible, since limit > 0) and are masked
  // afterwards, so all tiles' loads are in flight together.
  v4u raw[IS_TILES][4];
  float ks[IS_TILES];
  int pos[IS_TILES];
#pragma unroll
  for (int i = 0; i < IS_TILES; ++i) {
    const int tcol = col0 + (i * IS_WAVES + wave) * 32;
    pos[i] = (tcol < limit) ? column_position<POOL>(a, t, tcol + r, nvis) : -1;
    const int64_t row = base + max(pos[i], 0);
    const v4u* src = (const v4u*)(a.k + row * a.k_row_stride + 64 * half);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[i][j] = src[j];
    ks[i] = a.k_scale[row * a.k_scale_stride];
  }

  // A operand widened to f16; gate of head r with the q scale folded in,
  // then the 16 heads this lane's accumulators hold.
  v8h qa[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qa[2 * j] = fp8x8_to_f16(qraw[j][0], qraw[j][1]);
    qa[2 * j + 1] = fp8x8_to_f16(qraw[j][2], qraw[j][3]);
  }
  g_r *= qs_r;
  float gate[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) gate[j] = __shfl(g_r, 8 * (j >> 2) + 4 * half + (j & 3));

#pragma unroll
  for (int i = 0; i < IS_TILES; ++i) {
    const int tcol = col0 + (i * IS_WAVES + wave) * 32;
    if (tcol >= a.n_cols) break;
    const int col = tcol + r;
    float sc = -INFINITY;
    if (tcol < limit) {
      v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8h b0 = fp8x8_to_f16(raw[i][j][0], raw[i][j][1]);
        const v8h b1 = fp8x8_to_f16(raw[i][j][2], raw[i][j][3]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[2 * j], b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[2 * j + 1], b1, acc, 0, 0, 0);
      }
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) v = fmaf(gate[j], fmaxf(acc[j], 0.f), v);
      v += __shfl_xor(v, 32);
      sc = (pos[i] >= 0) ? v * ks[i] : -INFINITY;
    }
    if (half == 0 && col < a.n_cols) out[col] = sc;
    if (!POOL && a.block_max) {
      // maximum over aligned groups of block_size lanes (block_size <= 32)
      float m = sc;
      for (int sh = 1; sh < (1 << a.block_shift); sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
      if (half == 0 && (r & ((1 << a.block_shift) - 1)) == 0 && col < a.n_cols)
        a.block_max[(int64_t)t * a.block_max_stride + (col >> a.block_shift)] = m;
    }
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
  float* out = a.scores + (int64_t)t * a.score_stride;
  const int p = column_position<POOL>(a, t, col, nvis);
  float tot = -INFINITY;
  if (p >= 0) {
    const float* krow = (const float*)(a.k + (base + p) * a.k_row_stride);
    float kv[128];
#pragma unroll
    for (int d = 0; d < 128; d += 4) {
      const float4 x = *(const float4*)(krow + d);
      kv[d] = x.x; kv[d + 1] = x.y; kv[d + 2] = x.z; kv[d + 3] = x.w;
    }
    tot = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 128; ++d) dot = fmaf(sq[h * 128 + d], kv[d], dot);
      tot = fmaf(sw[h], fmaxf(dot, 0.f), tot);
    }
  }
  if (col < a.n_cols) out[col] = tot;
  if (!POOL && a.block_max) {
    // 256 consecutive columns per workgroup: wave-level groups of block_size
    float m = tot;
    for (int sh = 1; sh < (1 << a.block_shift); sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
    if ((threadIdx.x & ((1 << a.block_shift) - 1)) == 0 && col < a.n_cols)
      a.block_max[(int64_t)t * a.block_max_stride + (col >> a.block_shift)] = m;
  }
}

hipError_t launch_index_scores_fp8(const IndexScoreArgs& a, hipStream_t s) {
  dim3 grid((a.n_cols + IS_KEYS_PER_WG - 1) / IS_KEYS_PER_WG, a.Q);
  if (a.cand) {
    if (a.w_bf16)
      hipLaunchKernelGGL((index_scores_fp8_kernel<true, true>), grid, dim3(64 * IS_WAVES), 0, s, a);
    else
      hipLaunchKernelGGL((index_scores_fp8_kernel<true, false>), grid, dim3(64 * IS_WAVES), 0, s, a);
  } else {
    if (a.w_bf16)
      hipLaunchKernelGGL((index_scores_fp8_kernel<false, true>), grid, dim3(64 * IS_WAVES), 0, s, a);
    else
      hipLaunchKernelGGL((index_scores_fp8_kernel<false, false>), grid, dim3(64 * IS_WAVES), 0, s, a);
  }
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
