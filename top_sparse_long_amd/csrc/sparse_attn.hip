// Core sparse attention of the CSA2 hot path on gfx950.
//
// For query t and head i the keys are the layer's SWA rows of the window
// [max(lo, p - W + 1), p] followed by the top-k main rows; K = V (MQA, one
// 512-dim vector per key); one softmax per head over all of them, with a sink
// logit that enters only the denominator (CSA2 page, "per-layer attention
// computation"):
//     out = sum_j e^{z_j} K_j / (sum_j e^{z_j} + e^{sink_i}),  z_j = scale q.K_j
//
// Quantized path (bf16 q, FP4 main KV with 16 fp32 scales per row, FP8 SWA
// with 4 fp32 scales per row):
//   * one workgroup = one query x 16 heads; 4 waves split the key tiles
//     (32 keys each); the workgroups of a query sit on one XCD so its
//     gathered rows are shared through that XCD's L2;
//   * rows are gathered straight from HBM into registers, dequantized to f16
//     (exact E2M1/E4M3 codes times the scale, one f16 rounding), used at once
//     as the K operand of S^T = K Q^T on v_mfma_f32_16x16x32_f16, and written
//     to the wave's LDS tile for the P V product, which needs the same data
//     with keys along the reduction axis;
//   * S^T's accumulator layout puts 8 keys of one head in each lane, which is
//     exactly P's operand layout for P V, so the probabilities never move;
//   * online softmax in base 2 with lazy rescaling: the running maximum is
//     only raised when a tile's maximum exceeds it by more than 8 (so
//     probabilities stay below 2^8 in f16), and the four waves' partial
//     results are merged through LDS at the end.
// q is converted from bf16 to f16 (exact for |q| in the f16 normal range),
// so operands carry 11 significant bits; accumulation is fp32.
#include "kernels.h"

namespace csa2 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
struct v8s_pair {
  v4s_t lo, hi;
};

constexpr int AT_WAVES = 4;
constexpr int AT_HEADS = 16;
constexpr int AT_D = 512;
constexpr int AT_RS = AT_D * 2 + 16;          // LDS row stride (bytes) of an f16 key row
constexpr int AT_TILE_BYTES = 32 * AT_RS;     // one wave's 32-key tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.0f;         // log2 units

__device__ __forceinline__ uint32_t as_u32(v2h h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ v2h as_v2h(uint32_t u) { return __builtin_bit_cast(v2h, u); }

// Dequantization: gfx950's scaled converts (v_cvt_scalef32_pk_f16_fp4/fp8)
// widen two codes to f16 and apply only the exponent of their fp32 scale
// operand (a scale s acts as 2^floor(log2 s)).  The remaining mantissa factor
// m = s / 2^floor(log2 s), in [1, 2), is applied with one packed f16
// multiply, so value = code * s with a single f16 rounding of the product
// (plus the rounding of m to f16).
__device__ __forceinline__ _Float16 scale_mantissa(float s) {
  return (_Float16)(2.0f * __builtin_amdgcn_frexp_mantf(s));
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i).
__device__ __forceinline__ void dequant_fp4x8(uint32_t x, float s, v2h m2, uint32_t out[4]) {
  out[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, s, 0) * m2);
  out[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, s, 1) * m2);
  out[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, s, 2) * m2);
  out[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, s, 3) * m2);
}

// Four E4M3 codes (one dword).
__device__ __forceinline__ void dequant_fp8x4(uint32_t x, float s, v2h m2, uint32_t out[2]) {
  out[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, s, false) * m2);
  out[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, s, true) * m2);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void sparse_attn_quant_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[AT_WAVES * AT_TILE_BYTES];
  __shared__ float s_m[AT_WAVES][AT_HEADS];
  __shared__ float s_l[AT_WAVES][AT_HEADS];
  __shared__ float s_f[AT_HEADS];

  const int n_hg = a.H / AT_HEADS;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // consecutive (query, head-group) pairs on one XCD: workgroups are handed
  // to the 8 XCDs round-robin
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int t = bid / n_hg;
  const int hg = bid - t * n_hg;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;

  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  const int nvis = (int)(((int64_t)p + 1) / a.ratio);
  const int64_t mbase = a.main_base[b];
  const int lo = a.swa_lo ? a.swa_lo[b] : 0;
  const int sp0 = a.swa_pos0[b];
  const int first = max(max(lo, sp0), max(0, p - a.window + 1));
  const int n_swa = max(0, p - first + 1);
  const int64_t sbase = a.swa_base[b] + (first - sp0);
  const int n_swa_tiles = (n_swa + 31) >> 5;
  const int n_tiles = n_swa_tiles + ((a.k + 31) >> 5);

  // q as the B operand of S^T = K Q^T: head (16 hg + r), dims [128 g, +128),
  // chunk c holding dims 128 g + 8 c .. +8.
  v8h qf[16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t * a.H + hg * AT_HEADS + r) * AT_D + 128 * g;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const v4u raw = *(const v4u*)(qrow + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[c][2 * e] = (_Float16)__uint_as_float(raw[e] << 16);
        qf[c][2 * e + 1] = (_Float16)__uint_as_float(raw[e] & 0xFFFF0000u);
      }
    }
  }

  // O[T]: output columns d = 16 T + r, rows = heads 4 g + j
  v4f O[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) O[u] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_s = -INFINITY;   // running maximum of head r (log2 units)
  float l_part = 0.f;      // this lane's share of the denominator of head r
  const float zscale = a.scale * LOG2E;
  uint8_t* tile = s_tile + wave * AT_TILE_BYTES;

  for (int ti = wave; ti < n_tiles; ti += AT_WAVES) {
    const bool is_swa = ti < n_swa_tiles;
    const int slot0 = (is_swa ? ti : ti - n_swa_tiles) * 32;
    v4f acc[2];
    uint64_t vmask[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int slot = slot0 + kh * 16 + r;
      bool valid;
      int64_t row;
      if (is_swa) {
        valid = slot < n_swa;
        row = sbase + slot;
      } else {
        const int pos = slot < a.k ? a.idx[(int64_t)t * a.k + slot] : -1;
        valid = pos >= 0 && pos < nvis;
        row = mbase + pos;
      }
      vmask[kh] = __ballot(valid);
      uint32_t kd[16][4];   // chunk c: dims 128 g + 8 c .. +8 as f16 pairs
      if (is_swa) {
        v4u raw[8];
        float sc = 0.f;
        if (valid) {
          const uint8_t* src = a.swa + row * a.swa_stride + 128 * g;
#pragma unroll
          for (int j = 0; j < 8; ++j) raw[j] = *(const v4u*)(src + 16 * j);
          sc = a.swa_scale[row * a.swa_scale_stride + g];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) raw[j] = (v4u){0u, 0u, 0u, 0u};
        }
        const _Float16 mh = scale_mantissa(sc);
        const v2h m2 = {mh, mh};
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          dequant_fp8x4(raw[c >> 1][(c & 1) * 2], sc, m2, &kd[c][0]);
          dequant_fp8x4(raw[c >> 1][(c & 1) * 2 + 1], sc, m2, &kd[c][2]);
        }
      } else {
        v4u raw[4];
        float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
          const uint8_t* src = a.main + row * a.main_stride + 64 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) raw[j] = *(const v4u*)(src + 16 * j);
          sc = *(const float4*)(a.main_scale + row * a.main_scale_stride + 4 * g);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) raw[j] = (v4u){0u, 0u, 0u, 0u};
        }
        const float s4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const _Float16 mh = scale_mantissa(s4[c >> 2]);
          dequant_fp4x8(raw[c >> 2][c & 3], s4[c >> 2], (v2h){mh, mh}, kd[c]);
        }
      }
      // S^T for keys kh*16 .. +16 and the 16 heads
      v4f s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const v4u kv = {kd[c][0], kd[c][1], kd[c][2], kd[c][3]};
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qf[c], s, 0, 0, 0);
      }
      acc[kh] = s;
      // stage the dequantized row for P V
      uint8_t* dst = tile + (kh * 16 + r) * AT_RS + 256 * g;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const v4u kv = {kd[c][0], kd[c][1], kd[c][2], kd[c][3]};
        *(v4u*)(dst + 16 * c) = kv;
      }
    }

    // scores of head r for keys {4g+i} and {16+4g+i}
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ((vmask[0] >> (4 * g + i)) & 1ull) ? acc[0][i] * zscale : -INFINITY;
      z[4 + i] = ((vmask[1] >> (4 * g + i)) & 1ull) ? acc[1][i] * zscale : -INFINITY;
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool raise = mt > m_s + RESCALE_SLACK || (m_s == -INFINITY && mt > -INFINITY);
    if (__any(raise)) {
      const float m_new = fmaxf(m_s, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_s - m_new);
      l_part *= alpha;
      m_s = m_new;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * g + j);
#pragma unroll
        for (int u = 0; u < 32; ++u) O[u][j] *= aj;
      }
    }
    v8h P;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m_s);
      l_part += pv;
      P[i] = (_Float16)pv;
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O[h, d] += sum_keys P[h, key] V[key, d].  V is read transposed with
    // ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
    // i % 4 of the 8-byte rows addressed by lanes 4 j + i / 4 (j = 0..3).  Lane
    // (r, g) addresses key 4 g + r / 4 (then 16 + 4 g + r / 4) at column
    // 16 T + 4 (r % 4), so it receives V[4 g + j][16 T + r] (then the keys
    // 16 + 4 g + j): exactly its B operand for output columns 16 T .. +16.
    {
      __attribute__((address_space(3))) uint8_t* tl =
          (__attribute__((address_space(3))) uint8_t*)tile;
      const int off_a = (4 * g + (r >> 2)) * AT_RS + 8 * (r & 3);
      const int off_b = (16 + 4 * g + (r >> 2)) * AT_RS + 8 * (r & 3);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s_t*)(tl + off_a + 32 * u));
        const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s_t*)(tl + off_b + 32 * u));
        const v8s_pair pr = {lo, hi};
        const v8h bv = __builtin_bit_cast(v8h, pr);
        O[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, bv, O[u], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves ------------------------------------------------
  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g == 0) {
    s_m[wave][r] = m_s;
    s_l[wave][r] = l;
  }
  __syncthreads();
  const int h_glob0 = hg * AT_HEADS;
  if (threadIdx.x < AT_HEADS) {
    const int h = threadIdx.x;
    const float sink2 = a.sink[h_glob0 + h] * LOG2E;
    float M = sink2;
    for (int w = 0; w < AT_WAVES; ++w) M = fmaxf(M, s_m[w][h]);
    float den = (M == -INFINITY) ? 0.f : exp2f(sink2 - M);
    for (int w = 0; w < AT_WAVES; ++w)
      if (s_m[w][h] > -INFINITY) den += s_l[w][h] * exp2f(s_m[w][h] - M);
    s_f[h] = (den > 0.f) ? 1.f / den : 0.f;
    if (a.lse) a.lse[(int64_t)t * a.H + h_glob0 + h] = (M + log2f(den)) * LN2;
  }
  __syncthreads();
  // factor of this wave for the rows it holds: heads 4g + j
  float fw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    const float sink2 = a.sink[h_glob0 + h] * LOG2E;
    float M = sink2;
    for (int w = 0; w < AT_WAVES; ++w) M = fmaxf(M, s_m[w][h]);
    const float mw = s_m[wave][h];
    fw[j] = (mw == -INFINITY) ? 0.f : exp2f(mw - M) * s_f[h];
  }
  // each wave writes its scaled partial output (fp32 [16][512]) over its tile
  float* part = (float*)tile;
#pragma unroll
  for (int u = 0; u < 32; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) part[(4 * g + j) * AT_D + 16 * u + r] = O[u][j] * fw[j];
  __syncthreads();
  const float* p0 = (const float*)(s_tile + 0 * AT_TILE_BYTES);
  const float* p1 = (const float*)(s_tile + 1 * AT_TILE_BYTES);
  const float* p2 = (const float*)(s_tile + 2 * AT_TILE_BYTES);
  const float* p3 = (const float*)(s_tile + 3 * AT_TILE_BYTES);
  const int64_t obase = ((int64_t)t * a.H + h_glob0) * AT_D;
  for (int e = threadIdx.x * 4; e < AT_HEADS * AT_D; e += 256 * 4) {
    const float4 x0 = *(const float4*)(p0 + e);
    const float4 x1 = *(const float4*)(p1 + e);
    const float4 x2 = *(const float4*)(p2 + e);
    const float4 x3 = *(const float4*)(p3 + e);
    const float4 v = make_float4(x0.x + x1.x + x2.x + x3.x, x0.y + x1.y + x2.y + x3.y,
                                 x0.z + x1.z + x2.z + x3.z, x0.w + x1.w + x2.w + x3.w);
    if (a.out_bf16) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
      pk.y = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
      *(uint2*)((uint16_t*)a.out + obase + e) = pk;
    } else {
      *(float4*)((float*)a.out + obase + e) = v;
    }
  }
}

// fp32 path: one workgroup per (query, head); plain loops.
constexpr int AF_MAX_SLOTS = 8192;

__global__ __launch_bounds__(256) void sparse_attn_f32_kernel(AttnArgs a) {
  __shared__ float sq[AT_D];
  __shared__ float sz[AF_MAX_SLOTS];
  __shared__ float red[256];
  const int t = blockIdx.x / a.H;
  const int h = blockIdx.x - t * a.H;
  const int tid = threadIdx.x;
  const float* qrow = (const float*)a.q + ((int64_t)t * a.H + h) * AT_D;
  for (int d = tid; d < AT_D; d += 256) sq[d] = qrow[d];
  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  const int nvis = (int)(((int64_t)p + 1) / a.ratio);
  const int64_t mbase = a.main_base[b];
  const int lo = a.swa_lo ? a.swa_lo[b] : 0;
  const int sp0 = a.swa_pos0[b];
  const int first = max(max(lo, sp0), max(0, p - a.window + 1));
  const int n_swa = max(0, p - first + 1);
  const int64_t sbase = a.swa_base[b] + (first - sp0);
  const int n_slots = n_swa + a.k;
  __syncthreads();

  auto key_row = [&](int j) -> const float* {
    if (j < n_swa) return (const float*)(a.swa + (sbase + j) * a.swa_stride);
    const int pos = a.idx[(int64_t)t * a.k + (j - n_swa)];
    if (pos < 0 || pos >= nvis) return nullptr;
    return (const float*)(a.main + (mbase + pos) * a.main_stride);
  };

  float mx = -INFINITY;
  for (int j = tid; j < n_slots; j += 256) {
    const float* kr = key_row(j);
    float z = -INFINITY;
    if (kr) {
      float dot = 0.f;
      for (int d = 0; d < AT_D; ++d) dot = fmaf(sq[d], kr[d], dot);
      z = dot * a.scale;
    }
    sz[j] = z;
    mx = fmaxf(mx, z);
  }
  red[tid] = mx;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
    __syncthreads();
  }
  const float sink = a.sink[h];
  const float M = fmaxf(red[0], sink);
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < n_slots; j += 256) {
    const float e = (sz[j] == -INFINITY) ? 0.f : expf(sz[j] - M);
    sz[j] = e;
    sum += e;
  }
  red[tid] = sum;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  const float den = red[0] + ((M == -INFINITY) ? 0.f : expf(sink - M));
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int d = tid; d < AT_D; d += 256) {
    float acc = 0.f;
    for (int j = 0; j < n_slots; ++j) {
      const float e = sz[j];
      if (e == 0.f) continue;
      acc = fmaf(e, key_row(j)[d], acc);
    }
    ((float*)a.out)[((int64_t)t * a.H + h) * AT_D + d] = acc * inv;
  }
  if (tid == 0 && a.lse) a.lse[(int64_t)t * a.H + h] = M + logf(den);
}

hipError_t launch_sparse_attn_quant(const AttnArgs& a, hipStream_t s) {
  const int nblk = a.Q * (a.H / AT_HEADS);
  hipLaunchKernelGGL(sparse_attn_quant_kernel, dim3(nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_attn_f32_kernel, dim3(a.Q * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
