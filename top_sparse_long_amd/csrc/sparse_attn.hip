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
//   * one workgroup = one query x 16 heads (x one key split at small
//     batches); 8 waves, two per SIMD, split the key tiles (16 keys each);
//     the workgroups of a query sit on one XCD so its gathered rows are
//     shared through that XCD's L2;
//   * rows are gathered straight from HBM into registers, dequantized to f16
//     (exact E2M1/E4M3 codes times the scale, one f16 rounding), used at once
//     as the K operand of S^T = K Q^T on v_mfma_f32_16x16x32_f16, and written
//     to the wave's LDS tile for the P V product, which needs the same data
//     with keys along the reduction axis;
//   * S^T's accumulator layout puts 4 keys of one head in each lane, which is
//     exactly P's operand layout for P V (v_mfma_f32_16x16x16_f16), so the
//     probabilities never move;
//   * online softmax in base 2 with lazy rescaling: the running maximum is
//     only raised when a tile's maximum exceeds it by more than 8 (so
//     probabilities stay below 2^8 in f16), and the eight waves' partial
//     results are merged through LDS at the end.
// q is converted from bf16 to f16 (exact for |q| in the f16 normal range),
// so operands carry 11 significant bits; accumulation is fp32.
#include "kernels.h"

#include <type_traits>

namespace csa2 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
struct v8s_pair {
  v4s_t lo, hi;
};

constexpr int AT_HEADS = 16;
constexpr int AT_D = 512;
constexpr int AT_RS = AT_D * 2 + 16;          // LDS row stride (bytes) of an f16 key row
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.0f;         // log2 units
constexpr int AT_MAX_K = 2048;                // largest top-k the kernel stages

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

// Eight E2M1 codes times an E4M3 scale widened to f16: exact (a code has at
// most 2 significant bits, an E4M3 scale at most 4).
__device__ __forceinline__ void dequant_fp4x8_h(uint32_t x, _Float16 s, uint32_t out[4]) {
  const v2h s2 = {s, s};
  out[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2);
  out[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2);
  out[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2);
  out[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2);
}

// Four E4M3 codes (one dword).
__device__ __forceinline__ void dequant_fp8x4(uint32_t x, float s, v2h m2, uint32_t out[2]) {
  out[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, s, false) * m2);
  out[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, s, true) * m2);
}

// Inverse RoPE of one output pair (x, y) = dims (2i, 2i+1) of the turned
// range: x' = x cos + y sin, y' = y cos - x sin.
__device__ __forceinline__ void unturn(float& x, float& y, float c, float s) {
  const float x0 = x, y0 = y;
  x = x0 * c + y0 * s;
  y = y0 * c - x0 * s;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// One workgroup = one query x 16 heads (x one key split), eight waves over
// 16-key tiles (SWA tiles first), two waves per SIMD.  q is staged once in LDS
// as f16 and read per 8-dim chunk as
// the B operand of S^T = K Q^T, so a wave holds only O (128 registers), one
// tile's raw bytes and its working set, and two waves share each SIMD.  P V
// runs on v_mfma_f32_16x16x16_f16, whose A operand is S^T's accumulator
// layout for 16 keys (lane (r, g): head r, keys 4 g .. 4 g + 3) and whose B
// operand is what ds_read_b64_tr_b16 returns from the tile.  The eight
// waves' partial results are merged through LDS, one half of the 512 output
// columns at a time, into the output or (key splits) a partial record.
// (A four-wave form with 32-key tiles and q in registers needed ~500
// registers, one wave per SIMD: 26.3 us per 64-query group call against
// 21.9 us here, and 1.41 ms against 1.18 ms on the 4,096-query chunk.)
constexpr int AW_WAVES = 8;
constexpr int V3_RS = 528;                                     // LDS row stride of raw key bytes
constexpr int V3_SG = 32;                                      // scale groups staged per key (max)
constexpr int V3_QS = AT_D * 2 + 16;                           // LDS row stride of staged f16 q (bytes)
// LDS byte offset of raw key row `row` of a round: every 16-row block is
// shifted by 8 bytes, so the transposing reads of two 16-lane groups (two
// different 16-row blocks at the same column) use disjoint banks.
__device__ __forceinline__ int v3_row(int row) { return row * V3_RS + (row >> 4) * 8; }
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
constexpr int AW_TILE_BYTES = 16 * AT_RS;     // one wave's 16-key tile
static_assert(AW_WAVES * AW_TILE_BYTES >= AW_WAVES * 16 * 64 * 16, "half of every wave's O must fit the tiles");

template <bool S16, bool TURN>
__global__ __launch_bounds__(64 * AW_WAVES) void sparse_attn_quant_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[AW_WAVES * AW_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[AT_HEADS * AT_RS];
  __shared__ float s_m[AW_WAVES][AT_HEADS];
  __shared__ float s_l[AW_WAVES][AT_HEADS];
  __shared__ int32_t s_idx[AT_MAX_K];

  const int n_hg = a.H / AT_HEADS;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // the workgroups of a query on one XCD (handed out round-robin)
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int split = bid % a.n_split;
  const int tg = bid / a.n_split;
  const int t = tg / n_hg;
  const int hg = tg - t * n_hg;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;

  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  const int64_t lim = a.idx_slots ? a.n_main_rows : ((int64_t)p + 1) / a.ratio;
  const int64_t mbase = a.idx_slots ? 0 : a.main_base[b];
  const int lo = a.swa_lo ? a.swa_lo[b] : 0;
  const int sp0 = a.swa_pos0[b];
  const int first = max(max(lo, sp0), max(0, p - a.window + 1));
  const int n_swa = max(0, p - first + 1);
  const int64_t sbase = a.swa_base[b] + (first - sp0);
  const int n_swa_tiles = (n_swa + 15) >> 4;
  const int n_tiles_all = n_swa_tiles + ((a.k + 15) >> 4);
  // this workgroup's tiles: [tile_begin, n_tiles) of the query's tile list
  // (SWA tiles first); the whole list when keys are not split
  const int per_split = (n_tiles_all + a.n_split - 1) / a.n_split;
  const int tile_begin = min(n_tiles_all, split * per_split);
  const int n_tiles = min(n_tiles_all, tile_begin + per_split);
  const int h_glob0 = hg * AT_HEADS;
  // keys that do not exist are read from this query's own q row (always
  // mapped, 64 KB) and given a zero scale, so every load is unconditional
  const uint8_t* dummy = (const uint8_t*)a.q + (int64_t)t * a.H * AT_D * 2;

  // One 16-key tile as a lane holds it while the previous tile is computed:
  // key r of the tile, dims [128 g, +128).
  struct WSwa {
    v4u d[8];    // 128 E4M3 codes
    float s;     // the row's scale of these dims
    bool ok;
  };
  struct WMain {
    v4u d[4];    // 128 E2M1 codes
    float4 s;    // 4 fp32 scales, or 8 E4M3 scale bytes in the first two words
    bool ok;
  };
  auto load_swa = [&](int ti, WSwa& S) {
    const int slot = ti * 16 + r;
    // past the window's end: the last row again, masked later
    const int64_t row = sbase + min(slot, n_swa - 1);
    const uint8_t* src = a.swa + row * a.swa_stride + 128 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) S.d[j] = *(const v4u*)(src + 16 * j);
    S.s = a.swa_scale[row * a.swa_scale_stride + g];
    S.ok = slot < n_swa;
  };
  auto load_main = [&](int ti, WMain& M) {
    const int slot = (ti - n_swa_tiles) * 16 + r;
    const int pos = slot < a.k ? s_idx[slot] : -1;
    const bool v = pos >= 0 && pos < lim;
    const uint8_t* src = v ? a.main + (mbase + pos) * a.main_stride : dummy;
#pragma unroll
    for (int j = 0; j < 4; ++j) M.d[j] = *(const v4u*)(src + 64 * g + 16 * j);
    if (S16) {
      const uint8_t* ssrc = v ? (const uint8_t*)a.main_scale + (mbase + pos) * a.main_scale_stride : dummy;
      const uint2 sb = *(const uint2*)(ssrc + 8 * g);
      M.s = make_float4(__uint_as_float(sb.x), __uint_as_float(sb.y), 0.f, 0.f);
    } else {
      const float* ssrc = v ? a.main_scale + (mbase + pos) * a.main_scale_stride : (const float*)dummy;
      M.s = *(const float4*)(ssrc + 4 * g);
    }
    M.ok = v;
  };

  // ---- prologue: every independent load is issued before any is waited on
  WSwa S;
  WMain M;
  const int ti0 = tile_begin + wave;
  if (ti0 < n_tiles && ti0 < n_swa_tiles) load_swa(ti0, S);   // needs no staged index
  // q of the 16 heads: thread i converts dims [16 (i % 32), +16) of head i / 32
  v4u qraw[2];
  const int qh = threadIdx.x >> 5, qd = (threadIdx.x & 31) * 16;
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t * a.H + h_glob0 + qh) * AT_D + qd;
    qraw[0] = *(const v4u*)qrow;
    qraw[1] = *(const v4u*)(qrow + 8);
  }
  int32_t iv[AT_MAX_K / (64 * AW_WAVES)];
  if (a.k > 0) {
    const int32_t* irow = a.idx + (int64_t)t * a.k;
#pragma unroll
    for (int j = 0; j < AT_MAX_K / (64 * AW_WAVES); ++j)
      iv[j] = irow[min((int)threadIdx.x + 64 * AW_WAVES * j, a.k - 1)];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v8h h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[2 * e] = (_Float16)__uint_as_float(qraw[i][e] << 16);
      h[2 * e + 1] = (_Float16)__uint_as_float(qraw[i][e] & 0xFFFF0000u);
    }
    *(v8h*)(s_q + qh * AT_RS + 2 * qd + 16 * i) = h;
  }
  if (a.k > 0) {
#pragma unroll
    for (int j = 0; j < AT_MAX_K / (64 * AW_WAVES); ++j)
      if ((int)threadIdx.x + 64 * AW_WAVES * j < a.k) s_idx[threadIdx.x + 64 * AW_WAVES * j] = iv[j];
  }
  __syncthreads();   // s_q, s_idx
  if (ti0 >= n_swa_tiles && ti0 < n_tiles) load_main(ti0, M);

  // O[u]: output columns d = 16 u + r, rows = heads 4 g + j
  v4f O[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) O[u] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_s = -INFINITY;   // running maximum of head r (log2 units)
  float l_part = 0.f;      // this lane's share of the denominator of head r
  const float zscale = a.scale * LOG2E;
  uint8_t* tile = s_tile + wave * AW_TILE_BYTES;
  const uint8_t* qsrc = s_q + r * AT_RS + 256 * g;

  // S^T for the tile from dequantized 8-dim chunks (each also written to the
  // wave's LDS tile for P V) and q chunks read from LDS.
  auto stage_swa = [&](const WSwa& T, v4f& acc, uint64_t& vmask) {
    const _Float16 mh = scale_mantissa(T.s);
    const v2h m2 = {mh, mh};
    uint8_t* dst = tile + r * AT_RS + 256 * g;
    v4f s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      uint32_t kd[4];
      dequant_fp8x4(T.d[c >> 1][(c & 1) * 2], T.s, m2, &kd[0]);
      dequant_fp8x4(T.d[c >> 1][(c & 1) * 2 + 1], T.s, m2, &kd[2]);
      const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
      *(v4u*)(dst + 16 * c) = kv;
      const v8h qc = *(const v8h*)(qsrc + 16 * c);
      s2[c & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qc, s2[c & 1], 0, 0, 0);
    }
    acc = s2[0] + s2[1];
    vmask = __ballot(T.ok);
  };
  auto stage_main = [&](const WMain& T, v4f& acc, uint64_t& vmask) {
    const float4 sc = T.ok ? T.s : make_float4(0.f, 0.f, 0.f, 0.f);
    const float s4[4] = {sc.x, sc.y, sc.z, sc.w};
    _Float16 s8[8];
    if (S16) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const v2h lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__float_as_uint(s4[w]), 1.0f, false);
        const v2h hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__float_as_uint(s4[w]), 1.0f, true);
        s8[4 * w] = lo2[0];
        s8[4 * w + 1] = lo2[1];
        s8[4 * w + 2] = hi2[0];
        s8[4 * w + 3] = hi2[1];
      }
    }
    uint8_t* dst = tile + r * AT_RS + 256 * g;
    v4f s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      uint32_t kd[4];
      if (S16) {
        dequant_fp4x8_h(T.d[c >> 2][c & 3], s8[c >> 1], kd);
      } else {
        const _Float16 mh = scale_mantissa(s4[c >> 2]);
        dequant_fp4x8(T.d[c >> 2][c & 3], s4[c >> 2], (v2h){mh, mh}, kd);
      }
      const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
      *(v4u*)(dst + 16 * c) = kv;
      const v8h qc = *(const v8h*)(qsrc + 16 * c);
      s2[c & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qc, s2[c & 1], 0, 0, 0);
    }
    acc = s2[0] + s2[1];
    vmask = __ballot(T.ok);
  };

  // Online softmax over the tile's 16 scores of each head and O += P V.
  auto finish_tile = [&](const v4f acc, const uint64_t vmask) {
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = ((vmask >> (4 * g + i)) & 1ull) ? acc[i] * zscale : -INFINITY;
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
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
    v4h P;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m_s);
      l_part += pv;
      P[i] = (_Float16)pv;
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // lane (r, g) receives V[4 g + j][16 u + r] (j = 0..3): its B operand
    {
      __attribute__((address_space(3))) uint8_t* tl =
          (__attribute__((address_space(3))) uint8_t*)tile;
      const int off = (4 * g + (r >> 2)) * AT_RS + 8 * (r & 3);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const v4s_t vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s_t*)(tl + off + 32 * u));
        O[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, __builtin_bit_cast(v4h, vv), O[u], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // This wave's tiles are wave, wave + 8, ... (SWA tiles first); the next
  // tile's rows are requested once the current tile's bytes are staged.
  int ti = ti0;
  for (; ti < min(n_tiles, n_swa_tiles); ti += AW_WAVES) {
    v4f acc;
    uint64_t vmask;
    stage_swa(S, acc, vmask);
    const int nx = ti + AW_WAVES;
    if (nx < n_swa_tiles) load_swa(nx, S);
    else if (nx < n_tiles) load_main(nx, M);
    finish_tile(acc, vmask);
  }
  for (; ti < n_tiles; ti += AW_WAVES) {
    v4f acc;
    uint64_t vmask;
    stage_main(M, acc, vmask);
    if (ti + AW_WAVES < n_tiles) load_main(ti + AW_WAVES, M);
    finish_tile(acc, vmask);
  }

  // ---- merge the eight waves ----------------------------------------------
  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g == 0) {
    s_m[wave][r] = m_s;
    s_l[wave][r] = l;
  }
  __syncthreads();   // every wave is done with its tile; s_m, s_l
  constexpr int HALF_BYTES = 16 * 64 * 16;               // 16 column blocks of one wave
  if (a.n_split > 1) {
    // partial record of this split: per head the maximum over the waves
    // (log2 units, no sink), the denominator and O scaled onto that maximum
    float* rec = a.part + ((int64_t)tg * a.n_split + split) * ATTN_PART_FLOATS;
    float ew[AW_WAVES][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * g + j;
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < AW_WAVES; ++w) Mx = fmaxf(Mx, s_m[w][h]);
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < AW_WAVES; ++w) {
        const float mw = s_m[w][h];
        ew[w][j] = (mw == -INFINITY) ? 0.f : exp2f(mw - Mx);
        lsum += s_l[w][h] * ew[w][j];
      }
      if (wave == 0 && r == 0) {
        rec[h] = Mx;
        rec[16 + h] = lsum;
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint8_t* part = s_tile + wave * HALF_BYTES;
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) *(v4f*)(part + (uu * 64 + lane) * 16) = O[16 * half + uu];
      __syncthreads();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int uu = 2 * wave + k2;
        const int u = 16 * half + uu;
        v4f v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < AW_WAVES; ++w) {
          const v4f x = *(const v4f*)(s_tile + w * HALF_BYTES + (uu * 64 + lane) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] += x[j] * ew[w][j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) rec[32 + (4 * g + j) * AT_D + 16 * u + r] = v[j];
      }
      if (half == 0) __syncthreads();   // the second half reuses the tiles
    }
    return;
  }
  float fw[AW_WAVES][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    const float sink2 = a.sink[h_glob0 + h] * LOG2E;
    float Mx = sink2;
#pragma unroll
    for (int w = 0; w < AW_WAVES; ++w) Mx = fmaxf(Mx, s_m[w][h]);
    float den = (Mx == -INFINITY) ? 0.f : exp2f(sink2 - Mx);
#pragma unroll
    for (int w = 0; w < AW_WAVES; ++w) {
      const float mw = s_m[w][h];
      fw[w][j] = (mw == -INFINITY) ? 0.f : exp2f(mw - Mx);
      den += s_l[w][h] * fw[w][j];
    }
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
#pragma unroll
    for (int w = 0; w < AW_WAVES; ++w) fw[w][j] *= inv;
    if (a.lse && wave == 0 && r == 0) a.lse[(int64_t)t * a.H + h_glob0 + h] = (Mx + __builtin_amdgcn_logf(den)) * LN2;
  }
  const int64_t obase = ((int64_t)t * a.H + h_glob0 + 4 * g) * AT_D + r;
  // inverse RoPE of dims 448..511 (column blocks 28..31): the pair (2i, 2i+1)
  // sits in lanes r, r ^ 1, so a turning lane also merges its partner's column
  const bool turn = TURN && a.rope != nullptr && p >= 0 && p < a.n_rope;
  const float* cs = a.rope + (int64_t)max(p, 0) * 64;   // read only when turning
  constexpr int U_TURN = 28;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint8_t* part = s_tile + wave * HALF_BYTES;
#pragma unroll
    for (int uu = 0; uu < 16; ++uu) *(v4f*)(part + (uu * 64 + lane) * 16) = O[16 * half + uu];
    __syncthreads();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int uu = 2 * wave + k2;
      const int u = 16 * half + uu;
      v4f v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < AW_WAVES; ++w) {
        const v4f x = *(const v4f*)(s_tile + w * HALF_BYTES + (uu * 64 + lane) * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += x[j] * fw[w][j];
      }
      if (turn && u >= U_TURN) {
        v4f vp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < AW_WAVES; ++w) {
          const v4f x = *(const v4f*)(s_tile + w * HALF_BYTES + (uu * 64 + (lane ^ 1)) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) vp[j] += x[j] * fw[w][j];
        }
        const float c = cs[8 * (u - U_TURN) + (r >> 1)], sn = cs[32 + 8 * (u - U_TURN) + (r >> 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = (r & 1) ? vp[j] : v[j], y = (r & 1) ? v[j] : vp[j];
          unturn(x, y, c, sn);
          v[j] = (r & 1) ? y : x;
        }
      }
      // rows 4 g + j, column 16 u + r: 16 lanes write 16 consecutive columns
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t o = obase + (int64_t)j * AT_D + 16 * u;
        if (a.out_bf16) ((uint16_t*)a.out)[o] = f32_to_bf16_rne(v[j]);
        else ((float*)a.out)[o] = v[j];
      }
    }
    if (half == 0) __syncthreads();   // the second half reuses the tiles
  }
}

// ---------------------------------------------------------------------------
// Wide form for 64 heads: one workgroup = one query (x one key split), all
// 64 heads, eight waves (two per SIMD).  Heads are the M dimension of every
// product, so each gathered key row is dequantized once per query instead of
// once per 16-head group.  Keys go in rounds of 128 (SWA rounds first, then
// main rounds; a round holds keys of one format):
//
//   A  wave w takes keys 16 w .. 16 w + 15 of the round (raw bytes requested
//      into registers during the previous round's phase C): dequantized in
//      registers, they are the K operand of S^T = K Q^T for the four 16-head
//      blocks (q of all heads is staged once in LDS as f16).  The tile's
//      per-head maxima go to LDS;
//   B  after a barrier every wave forms the same running maxima (raised only
//      when a tile exceeds them by more than 8, so P < 2^8 in f16), writes
//      its tile's P, its keys' scales (f16, zero for keys that do not exist)
//      and its raw bytes to the round's LDS tile;
//   C  after a second barrier wave w owns columns 64 w .. 64 w + 63 for all
//      64 heads: one transposing read of the raw tile (ds_read_b64_tr_b4: 16
//      keys of one column per lane; ds_read_b64_tr_b8: 8 keys) widens
//      exactly to f16, is multiplied by the keys' scales, and feeds the P V
//      products of all four head blocks.
// The LDS tile is written in B and read in C, so one copy suffices: a wave
// writing round r + 1's tile has passed round r + 1's first barrier, which
// every wave reaches only after its phase C of round r.
constexpr int WD_WAVES = 8;
constexpr int WD_ROUND = 16 * WD_WAVES;                        // keys per round
constexpr int WD_RBUF = WD_ROUND * V3_RS + (WD_ROUND / 16) * 8;
constexpr int WD_PS = 2 * WD_ROUND + 16;                       // LDS row stride of P (bytes)
constexpr int WD_H = 64;
// batches of at least this many 64-head queries use the wide form (one
// workgroup per query fills the chip); smaller ones the 16-head groups
constexpr int WD_MIN_Q = 256;

template <bool S16, bool TURN>
__global__ __launch_bounds__(64 * WD_WAVES) void sparse_attn_wide_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_q[WD_H * V3_QS];
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[WD_RBUF];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[WD_H * WD_PS];
  __shared__ __attribute__((aligned(16))) _Float16 s_scl[V3_SG][WD_ROUND];
  __shared__ float s_m[WD_WAVES][WD_H];

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // the workgroups of a query on one XCD (handed out round-robin)
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int split = bid % a.n_split;
  const int t = bid / a.n_split;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;

  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  const int64_t lim = a.idx_slots ? a.n_main_rows : ((int64_t)p + 1) / a.ratio;
  const int64_t mbase = a.idx_slots ? 0 : a.main_base[b];
  const int lo = a.swa_lo ? a.swa_lo[b] : 0;
  const int sp0 = a.swa_pos0[b];
  const int first = max(max(lo, sp0), max(0, p - a.window + 1));
  const int n_swa = max(0, p - first + 1);
  const int64_t sbase = a.swa_base[b] + (first - sp0);
  const int n_swa_rounds = (n_swa + WD_ROUND - 1) / WD_ROUND;
  const int n_rounds = n_swa_rounds + (a.k + WD_ROUND - 1) / WD_ROUND;
  // this workgroup's rounds: [rb, re), the rounds dealt out evenly
  const int rb = (int)((int64_t)split * n_rounds / a.n_split);
  const int re = (int)((int64_t)(split + 1) * n_rounds / a.n_split);
  const int32_t* irow = a.idx + (int64_t)t * a.k;
  // keys that do not exist are read from this query's own q row (always
  // mapped, 64 KB) and get a zero scale and probability
  const uint8_t* dummy = (const uint8_t*)a.q + (int64_t)t * WD_H * AT_D * 2;

  struct Raw {
    v4u d[8];
    float4 s;
    bool ok;
  };
  // the main-KV position of lane (r, g)'s key in round rd (requested a round
  // ahead, so the row loads never wait on it)
  auto key_pos = [&](int rd) -> int {
    const int slot = (rd - n_swa_rounds) * WD_ROUND + 16 * wave + r;
    return (rd >= n_swa_rounds && slot < a.k) ? irow[slot] : -1;
  };
  // lane (r, g): key r of the wave's 16, dims [128 g, +128); pos from key_pos
  auto load_tile = [&](int rd, int pos, Raw& R) {
    if (rd < n_swa_rounds) {
      const int slot = rd * WD_ROUND + 16 * wave + r;
      const int64_t row = sbase + min(slot, max(n_swa - 1, 0));   // past the window: the last row again
      const uint8_t* src = a.swa + row * a.swa_stride + 128 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) R.d[j] = *(const v4u*)(src + 16 * j);
      R.s = make_float4(a.swa_scale[row * a.swa_scale_stride + g], 0.f, 0.f, 0.f);
      R.ok = slot < n_swa;
    } else {
      const bool v = pos >= 0 && pos < lim;
      const uint8_t* src = v ? a.main + (mbase + pos) * a.main_stride : dummy;
#pragma unroll
      for (int j = 0; j < 4; ++j) R.d[j] = *(const v4u*)(src + 64 * g + 16 * j);
      if (S16) {
        const uint8_t* ssrc = v ? (const uint8_t*)a.main_scale + (mbase + pos) * a.main_scale_stride : dummy;
        const uint2 sb = *(const uint2*)(ssrc + 8 * g);
        R.s = make_float4(__uint_as_float(sb.x), __uint_as_float(sb.y), 0.f, 0.f);
      } else {
        const float* ssrc = v ? a.main_scale + (mbase + pos) * a.main_scale_stride : (const float*)dummy;
        R.s = *(const float4*)(ssrc + 4 * g);
      }
      R.ok = v;
    }
  };

  // ---- prologue
  Raw R;
  if (rb < re) load_tile(rb, key_pos(rb), R);
  {
    // q of all heads to LDS as f16: thread i converts 64 consecutive dims
    const int qh = threadIdx.x >> 3, qd = (threadIdx.x & 7) * 64;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t * WD_H + qh) * AT_D + qd;
    v4u qraw[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qraw[c] = *(const v4u*)(qrow + 8 * c);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v8h h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[2 * e] = (_Float16)__uint_as_float(qraw[c][e] << 16);
        h[2 * e + 1] = (_Float16)__uint_as_float(qraw[c][e] & 0xFFFF0000u);
      }
      *(v8h*)(s_q + qh * V3_QS + 2 * qd + 16 * c) = h;
    }
  }
  float sink2[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) sink2[hb] = a.sink[16 * hb + r] * LOG2E;
  __syncthreads();   // s_q

  // O[hb][cb]: heads 16 hb + 4 g + j, column 64 wave + 16 cb + r
  v4f O[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[hb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_s[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // head 16 hb + r, log2 units
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};   // head 16 hb + r over this wave's keys
  const float zscale = a.scale * LOG2E;
  const int c0 = 64 * wave;
  const uint8_t* qsrc = s_q + r * V3_QS + 256 * g;

  // one round; SWA and main rounds are compiled apart so neither path keeps
  // the other's registers alive
  auto round = [&](auto swa_tag, int rd) {
    constexpr bool swa_round = decltype(swa_tag)::value;
    const int pos_next = (rd + 1 < re) ? key_pos(rd + 1) : -1;
    // ---- phase A: S^T of the wave's 16 keys for all 64 heads
    v4f acc[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc[hb] = (v4f){0.f, 0.f, 0.f, 0.f};
    if constexpr (swa_round) {
      const float sc = R.s.x;
      const _Float16 mh = scale_mantissa(sc);
      const v2h m2 = {mh, mh};
      // the q chunks of step c + 1 are read from LDS before the products of
      // step c; the scheduling barrier keeps the compiler from sinking each
      // read next to its product, which left one LDS round trip exposed per
      // product (4,096-query chunk: 622 -> 602 us per call)
      v8h qn[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        v8h qc[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) qc[hb] = qn[hb];
        if (c + 1 < 16) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS + 16 * (c + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        uint32_t kd[4];
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2], sc, m2, &kd[0]);
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2 + 1], sc, m2, &kd[2]);
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qc[hb], acc[hb], 0, 0, 0);
      }
    } else {
      const float s4[4] = {R.s.x, R.s.y, R.s.z, R.s.w};
      _Float16 s8[8];
      if (S16) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const v2h lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__float_as_uint(s4[w]), 1.0f, false);
          const v2h hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__float_as_uint(s4[w]), 1.0f, true);
          s8[4 * w] = lo2[0];
          s8[4 * w + 1] = lo2[1];
          s8[4 * w + 2] = hi2[0];
          s8[4 * w + 3] = hi2[1];
        }
      }
      v8h qn[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        v8h qc[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) qc[hb] = qn[hb];
        if (c + 1 < 16) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS + 16 * (c + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        uint32_t kd[4];
        if (S16) {
          dequant_fp4x8_h(R.d[c >> 2][c & 3], s8[c >> 1], kd);
        } else {
          const _Float16 mh = scale_mantissa(s4[c >> 2]);
          dequant_fp4x8(R.d[c >> 2][c & 3], s4[c >> 2], (v2h){mh, mh}, kd);
        }
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qc[hb], acc[hb], 0, 0, 0);
      }
    }
    // lane (r, g) of S^T holds keys 4 g + i of the tile for head 16 hb + r
    const uint64_t vmask = __ballot(R.ok);
    float z[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[hb][i] = ((vmask >> (4 * g + i)) & 1ull) ? acc[hb][i] * zscale : -INFINITY;
      float mt = fmaxf(fmaxf(z[hb][0], z[hb][1]), fmaxf(z[hb][2], z[hb][3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (g == 0) s_m[wave][4 * r + hb] = mt;
    }
    __syncthreads();

    // ---- phase B: running maxima (raised lazily, the same in every wave),
    // P, scales, raw bytes
    {
      bool raise = false;
      float alpha[4];
      // the maxima are stored [wave][r][head block]: one 16-byte read per wave
      v4f mx4 = *(const v4f*)(&s_m[0][4 * r]);
#pragma unroll
      for (int w = 1; w < WD_WAVES; ++w) {
        const v4f x = *(const v4f*)(&s_m[w][4 * r]);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) mx4[hb] = fmaxf(mx4[hb], x[hb]);
      }
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float mx = mx4[hb];
        const bool up = mx > m_s[hb] + RESCALE_SLACK || (m_s[hb] == -INFINITY && mx > -INFINITY);
        const float m_new = up ? mx : m_s[hb];
        alpha[hb] = (m_new == -INFINITY || !up) ? 1.f : __builtin_amdgcn_exp2f(m_s[hb] - m_new);
        raise |= up;
        m_s[hb] = m_new;
        // z - m_new <= 8 here, and -inf gives 0
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(z[hb][i] - m_new);
        l_part[hb] = l_part[hb] * alpha[hb] + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
        const v4h P4 = {(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
        *(v4h*)(s_p + (16 * hb + r) * WD_PS + 2 * (16 * wave + 4 * g)) = P4;
      }
      const float4 cs4 = R.ok ? R.s : make_float4(0.f, 0.f, 0.f, 0.f);
      const int key = 16 * wave + r;
      uint8_t* dst = s_raw + v3_row(key);
      if constexpr (swa_round) {
        s_scl[g][key] = (_Float16)cs4.x;
#pragma unroll
        for (int j = 0; j < 8; ++j) *(v4u*)(dst + 128 * g + 16 * j) = R.d[j];
      } else {
        if (S16) {
          const uint32_t w0 = __float_as_uint(cs4.x), w1 = __float_as_uint(cs4.y);
          const v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
          const v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
          const v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
          const v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
          s_scl[8 * g + 0][key] = a0[0];
          s_scl[8 * g + 1][key] = a0[1];
          s_scl[8 * g + 2][key] = a1[0];
          s_scl[8 * g + 3][key] = a1[1];
          s_scl[8 * g + 4][key] = a2[0];
          s_scl[8 * g + 5][key] = a2[1];
          s_scl[8 * g + 6][key] = a3[0];
          s_scl[8 * g + 7][key] = a3[1];
        } else {
          s_scl[4 * g + 0][key] = (_Float16)cs4.x;
          s_scl[4 * g + 1][key] = (_Float16)cs4.y;
          s_scl[4 * g + 2][key] = (_Float16)cs4.z;
          s_scl[4 * g + 3][key] = (_Float16)cs4.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *(v4u*)(dst + 64 * g + 16 * j) = R.d[j];
      }
      // every wave takes the same decision (same maxima, same rule)
      if (__any(raise)) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float aj = __shfl(alpha[hb], 4 * g + j);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) O[hb][cb][j] *= aj;
          }
        }
      }
    }
    __syncthreads();
    // the next round's rows (this round's bytes are in LDS now)
    if (rd + 1 < re) load_tile(rd + 1, pos_next, R);

    // ---- phase C: O[64 x 64] += P (V * scale) over the round's keys
    {
      const lds_u8* rawl = (const lds_u8*)s_raw;
      if constexpr (swa_round) {
        // 32-key blocks: lane group g holds keys 32 kb + 8 g .. + 7; the
        // wave's 64 columns lie in one 128-dim scale group.  The four column
        // blocks' V operands are widened first, then P streams by head block.
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int k0 = 32 * kb + 8 * g;
          const v8h S8 = *(const v8h*)(&s_scl[wave >> 1][k0]);
          const int rrow = v3_row(k0 + (r >> 1));
          v8h B[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const v2i_t tv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + c0 + 16 * cb + 8 * (r & 1)));
            const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, false);
            const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, true);
            const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, false);
            const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, true);
            B[cb] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]} * S8;
          }
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const v8h P = *(const v8h*)(s_p + (16 * hb + r) * WD_PS + 2 * k0);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, B[cb], O[hb][cb], 0, 0, 0);
          }
        }
      } else {
        // halves of 64 keys: lane group g holds tile 4 half + g (16 keys);
        // one transposing read gives those 16 keys of one column (keys 0..7
        // and 8..15 feed two products).  V operands first, then P by head block.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 16 * (4 * half + g);
          const int rrow = v3_row(kt + r);
          // every LDS read of the half (scales, transposing reads, the first
          // head block's P) is issued before the conversions, and each head
          // block's P is read during the previous block's products (602 ->
          // 596 us per call on the same chunk)
          v8h B1[4], B2[4];
          v8h S1s[4], S2s[4];
          v2i_t tvs[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int grp = S16 ? (4 * wave + cb) : (2 * wave + (cb >> 1));
            S1s[cb] = *(const v8h*)(&s_scl[grp][kt]);
            S2s[cb] = *(const v8h*)(&s_scl[grp][kt + 8]);
            tvs[cb] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + (c0 + 16 * cb) / 2));
          }
          v8h P1n = *(const v8h*)(s_p + r * WD_PS + 2 * kt);
          v8h P2n = *(const v8h*)(s_p + r * WD_PS + 2 * (kt + 8));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const v8h S1 = S1s[cb], S2 = S2s[cb];
            const v2i_t tv = tvs[cb];
            uint32_t b1[4], b2[4];
            b1[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[0], 1.0f, 0));
            b1[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[0], 1.0f, 1));
            b1[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[0], 1.0f, 2));
            b1[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[0], 1.0f, 3));
            b2[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[1], 1.0f, 0));
            b2[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[1], 1.0f, 1));
            b2[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[1], 1.0f, 2));
            b2[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)tv[1], 1.0f, 3));
            const v4u u1 = {b1[0], b1[1], b1[2], b1[3]}, u2 = {b2[0], b2[1], b2[2], b2[3]};
            B1[cb] = __builtin_bit_cast(v8h, u1) * S1;
            B2[cb] = __builtin_bit_cast(v8h, u2) * S2;
          }
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const v8h P1 = P1n, P2 = P2n;
            if (hb + 1 < 4) {
              P1n = *(const v8h*)(s_p + (16 * (hb + 1) + r) * WD_PS + 2 * kt);
              P2n = *(const v8h*)(s_p + (16 * (hb + 1) + r) * WD_PS + 2 * (kt + 8));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
              O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P1, B1[cb], O[hb][cb], 0, 0, 0);
              O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P2, B2[cb], O[hb][cb], 0, 0, 0);
            }
          }
        }
      }
    }
  };
  int rd = rb;
  for (; rd < min(re, n_swa_rounds); ++rd) round(std::true_type{}, rd);
  for (; rd < re; ++rd) round(std::false_type{}, rd);

  // ---- epilogue: denominators, sink, output (or partial records)
  __syncthreads();   // every wave is past its last read of s_m, s_raw and s_p
  // per head: the running maximum and this wave's denominator share, then
  // the row factors of O (heads 16 hb + 4 g + j) from LDS
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    float l = l_part[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (g == 0) s_m[wave][16 * hb + r] = l;
  }
  float* s_mx = (float*)s_p;   // [64] running maxima, [64] sink logits (log2 units)
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      s_mx[16 * hb + r] = m_s[hb];
      s_mx[64 + 16 * hb + r] = sink2[hb];
    }
  }
  __syncthreads();
  float Lh[4][4], Mh[4][4], Sk[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const v4f mv = *(const v4f*)(s_mx + 16 * hb + 4 * g);
    const v4f sv = *(const v4f*)(s_mx + 64 + 16 * hb + 4 * g);
    v4f L = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < WD_WAVES; ++w) L += *(const v4f*)(&s_m[w][16 * hb + 4 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Lh[hb][j] = L[j];
      Mh[hb][j] = mv[j];
      Sk[hb][j] = sv[j];
    }
  }
  if (a.n_split > 1) {
    // partial records, one per 16-head block (the layout the combine reads):
    // per head the running maximum (log2 units, no sink), the denominator and
    // O, all relative to that maximum
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      float* rec = a.part + (((int64_t)t * 4 + hb) * a.n_split + split) * ATTN_PART_FLOATS;
      if (wave == 0 && r == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rec[4 * g + j] = Mh[hb][j];
          rec[16 + 4 * g + j] = Lh[hb][j];
        }
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) rec[32 + (4 * g + j) * AT_D + c0 + 16 * cb + r] = O[hb][cb][j];
    }
    return;
  }
  float fo[4][4];
  const bool write_lse = a.lse && wave == 0 && r == 0;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sk = Sk[hb][j];
      const float Mx = fmaxf(Mh[hb][j], sk);
      const float e_keys = (Mh[hb][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mh[hb][j] - Mx);
      const float den = Lh[hb][j] * e_keys + ((Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sk - Mx));
      fo[hb][j] = (den > 0.f) ? e_keys * __builtin_amdgcn_rcpf(den) : 0.f;
      if (write_lse) a.lse[(int64_t)t * WD_H + 16 * hb + 4 * g + j] = (Mx + __builtin_amdgcn_logf(den)) * LN2;
    }
  // inverse RoPE of dims 448..511 (wave 7's columns): the pair (2i, 2i+1)
  // sits in lanes r, r ^ 1
  const bool turn = TURN && a.rope != nullptr && p >= 0 && p < a.n_rope && wave == 7;
  const float* cs = a.rope + (int64_t)max(p, 0) * 64;   // read only when turning
  // output through LDS (the raw tile is free), one 16-head block at a time:
  // each wave stages its 16 x 64 block, then every lane stores a 16-byte run
  constexpr int OSB = 64 * 4 + 16;                       // staged row stride (bytes), room for fp32
  static_assert(WD_WAVES * 16 * OSB <= WD_RBUF, "the staged output fits the raw tile");
  uint8_t* ob = s_raw + wave * 16 * OSB;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      v4f v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = O[hb][cb][j] * fo[hb][j];
      if (TURN) {
        v4f vp;
#pragma unroll
        for (int j = 0; j < 4; ++j) vp[j] = __shfl_xor(v[j], 1);
        if (turn) {
          const int i = (16 * cb + r) >> 1;
          const float c = cs[i], sn = cs[32 + i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x = (r & 1) ? vp[j] : v[j], y = (r & 1) ? v[j] : vp[j];
            unturn(x, y, c, sn);
            v[j] = (r & 1) ? y : x;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) *(float*)(ob + (4 * g + j) * OSB + 4 * (16 * cb + r)) = v[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 16 rows of 64 fp32 columns: bf16 out, 8 lanes x 8 columns per row
    // (hardware round-to-nearest-even conversion); fp32 out, 16 lanes x 4
    if (a.out_bf16) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int row = 8 * it + (lane >> 3);
        const v4f x0 = *(const v4f*)(ob + row * OSB + 32 * (lane & 7));
        const v4f x1 = *(const v4f*)(ob + row * OSB + 32 * (lane & 7) + 16);
        v4u pk;
        pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[1]) << 16);
        pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[3]) << 16);
        pk[2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[1]) << 16);
        pk[3] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[3]) << 16);
        const int64_t o = ((int64_t)t * WD_H + 16 * hb + row) * AT_D + c0 + 8 * (lane & 7);
        *(v4u*)((uint16_t*)a.out + o) = pk;
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = 4 * it + (lane >> 4);
        const v4u v = *(const v4u*)(ob + row * OSB + 16 * (lane & 15));
        const int64_t o = ((int64_t)t * WD_H + 16 * hb + row) * AT_D + c0 + 4 * (lane & 15);
        *(v4u*)((float*)a.out + o) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  const int64_t lim = a.idx_slots ? a.n_main_rows : ((int64_t)p + 1) / a.ratio;
  const int64_t mbase = a.idx_slots ? 0 : a.main_base[b];
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
    if (pos < 0 || pos >= lim) return nullptr;
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
  const bool turn = a.rope != nullptr && p >= 0 && p < a.n_rope;
  for (int d = tid; d < AT_D; d += 256) {
    float acc = 0.f;
    for (int j = 0; j < n_slots; ++j) {
      const float e = sz[j];
      if (e == 0.f) continue;
      acc = fmaf(e, key_row(j)[d], acc);
    }
    float o = acc * inv;
    if (turn && d >= 448) {   // whole waves: threads 192..255 in the second pass
      const float other = __shfl_xor(o, 1);
      const int i = (d - 448) >> 1;
      const float c = a.rope[(int64_t)p * 64 + i], sn = a.rope[(int64_t)p * 64 + 32 + i];
      float x = (d & 1) ? other : o, y = (d & 1) ? o : other;
      unturn(x, y, c, sn);
      o = (d & 1) ? y : x;
    }
    ((float*)a.out)[((int64_t)t * a.H + h) * AT_D + d] = o;
  }
  if (tid == 0 && a.lse) a.lse[(int64_t)t * a.H + h] = M + logf(den);
}

// Combine the partial records of the key splits of one (query, 16 heads):
// the common maximum includes the sink, which enters only the denominator.
// ATTN_COMBINE_PARTS workgroups of ATTN_COMBINE_THREADS threads per (query,
// 16 heads), one 4-column group per thread, so the partial records are read
// by many CUs at once (measured: 8 x 256 threads is 0.7 us faster per call
// than 4 x 256 with two groups per thread); every load (all splits' partial
// O and their m, l) is issued before any is used, so one memory round trip
// covers the combine.
constexpr int ATTN_MAX_SPLIT = 16;

#ifndef CSA2_COMBINE_PARTS
#define CSA2_COMBINE_PARTS 8
#endif
constexpr int ATTN_COMBINE_PARTS = CSA2_COMBINE_PARTS;
constexpr int ATTN_COMBINE_THREADS = AT_HEADS * AT_D / ATTN_COMBINE_PARTS / 4;
static_assert(ATTN_COMBINE_THREADS * ATTN_COMBINE_PARTS * 4 == AT_HEADS * AT_D &&
              ATTN_COMBINE_THREADS % 64 == 0 && ATTN_COMBINE_THREADS <= 1024,
              "one 4-column group per thread");

// NS = the number of splits (compiled per count, so a thread issues exactly
// one record read per split).
template <int NS>
__global__ __launch_bounds__(ATTN_COMBINE_THREADS) void sparse_attn_combine_kernel(AttnArgs a) {
  const int n_hg = a.H / AT_HEADS;
  const int tg = blockIdx.x / ATTN_COMBINE_PARTS;
  const int e0 = (blockIdx.x % ATTN_COMBINE_PARTS) * (AT_HEADS * AT_D / ATTN_COMBINE_PARTS);
  const int t = tg / n_hg;
  const int h0 = (tg - t * n_hg) * AT_HEADS;
  const float* rec0 = a.part + (int64_t)tg * NS * ATTN_PART_FLOATS;
  float4 x[1][NS];
  float ms[1][NS], ls[1][NS];
#pragma unroll
  for (int i = 0; i < 1; ++i) {
    const int e = e0 + threadIdx.x * 4;
    const int h = e / AT_D;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const float* rec = rec0 + sp * ATTN_PART_FLOATS;
      x[i][sp] = *(const float4*)(rec + 32 + e);
      ms[i][sp] = rec[h];
      ls[i][sp] = rec[16 + h];
    }
  }
  const int64_t obase = ((int64_t)t * a.H + h0) * AT_D;
  // inverse RoPE of dims 448..511: a thread's four columns are two pairs
  const int p = a.rope ? a.q_pos[t] : 0;
  const bool turn = a.rope != nullptr && p >= 0 && p < a.n_rope;
#pragma unroll
  for (int i = 0; i < 1; ++i) {
    const int e = e0 + threadIdx.x * 4;
    const int h = e / AT_D;
    const float sink2 = a.sink[h0 + h] * LOG2E;
    float M = sink2;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) M = fmaxf(M, ms[i][sp]);
    float den = (M == -INFINITY) ? 0.f : exp2f(sink2 - M);
    float f[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      f[sp] = (ms[i][sp] == -INFINITY) ? 0.f : exp2f(ms[i][sp] - M);
      den += ls[i][sp] * f[sp];
    }
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const float fs = f[sp] * inv;
      v.x += x[i][sp].x * fs;
      v.y += x[i][sp].y * fs;
      v.z += x[i][sp].z * fs;
      v.w += x[i][sp].w * fs;
    }
    if (a.lse && (e % AT_D) == 0) a.lse[(int64_t)t * a.H + h0 + h] = (M + __builtin_amdgcn_logf(den)) * LN2;
    const int col = e % AT_D;
    if (turn && col >= 448) {
      const float* cs = a.rope + (int64_t)p * 64 + ((col - 448) >> 1);
      unturn(v.x, v.y, cs[0], cs[32]);
      unturn(v.z, v.w, cs[1], cs[33]);
    }
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

template <int NS>
static void launch_combine_n(const AttnArgs& a, int groups, hipStream_t s) {
  hipLaunchKernelGGL((sparse_attn_combine_kernel<NS>), dim3(groups * ATTN_COMBINE_PARTS),
                     dim3(ATTN_COMBINE_THREADS), 0, s, a);
}

template <int NS>
static void launch_combine_upto(const AttnArgs& a, int groups, hipStream_t s) {
  if constexpr (NS >= 2) {
    if (a.n_split == NS) launch_combine_n<NS>(a, groups, s);
    else launch_combine_upto<NS - 1>(a, groups, s);
  }
}

static void launch_combine(const AttnArgs& a, int groups, hipStream_t s) {
  launch_combine_upto<ATTN_MAX_SPLIT>(a, groups, s);
}

// Key splits per (query, 16 heads): only when the batch leaves most of the
// chip idle; about eight 16-key tiles per split (one per wave), at most 8.
int attn_splits(int Q, int H, int k, int window) {
  if (Q <= 0) return 1;
  if (H == WD_H && Q >= WD_MIN_Q) return 1;   // wide form, one workgroup per query
  const int groups = Q * (H / AT_HEADS);
  if (groups <= 0 || groups >= 128) return 1;
  const int tiles = (window + 15) / 16 + (k + 15) / 16;   // 16-key tiles
  int ns = (tiles + AW_WAVES - 1) / AW_WAVES;             // about one per wave
  ns = min(ns, max(1, 256 / groups));
  return max(1, min(ns, ATTN_MAX_SPLIT));
}

hipError_t launch_sparse_attn_quant(const AttnArgs& a, hipStream_t s) {
  const int groups = a.Q * (a.H / AT_HEADS);
  if (a.H == WD_H && a.Q >= WD_MIN_Q) {
    // split calls turn the output in the combine kernel
    const bool turn = a.rope != nullptr && a.n_split == 1;
    const dim3 grid(a.Q * a.n_split), block(64 * WD_WAVES);
    if (a.main_s16) {
      if (turn) hipLaunchKernelGGL((sparse_attn_wide_kernel<true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((sparse_attn_wide_kernel<true, false>), grid, block, 0, s, a);
    } else {
      if (turn) hipLaunchKernelGGL((sparse_attn_wide_kernel<false, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((sparse_attn_wide_kernel<false, false>), grid, block, 0, s, a);
    }
    if (a.n_split > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      launch_combine(a, groups, s);
    }
    return hipGetLastError();
  }
  // split calls turn the output in the combine kernel
  const bool turn = a.rope != nullptr && a.n_split == 1;
  const dim3 grid(groups * a.n_split), block(64 * AW_WAVES);
  if (a.main_s16) {
    if (turn) hipLaunchKernelGGL((sparse_attn_quant_kernel<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sparse_attn_quant_kernel<true, false>), grid, block, 0, s, a);
  } else {
    if (turn) hipLaunchKernelGGL((sparse_attn_quant_kernel<false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sparse_attn_quant_kernel<false, false>), grid, block, 0, s, a);
  }
  if (a.n_split > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_combine(a, groups, s);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_attn_f32_kernel, dim3(a.Q * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
