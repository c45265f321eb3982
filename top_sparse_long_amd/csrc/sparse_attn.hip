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
// with 4 fp32 scales per row), two kernels of one design:
//   * heads are the M dimension of every product: a workgroup takes one
//     query and 64 heads (large batches) or 16 heads and a part of the
//     output columns (everything else), so each gathered row is dequantized
//     once per workgroup; the workgroups of a query sit on one XCD, so its
//     rows come from HBM once and are shared through that XCD's L2;
//   * keys go in rounds of 128, 16 per wave: a wave dequantizes its rows in
//     registers to f16 (exact E2M1/E4M3 codes times the scale, one f16
//     rounding) as the K operand of S^T = K Q^T on v_mfma_f32_16x16x32_f16
//     and stores the raw bytes in LDS; S^T's accumulator layout (4 keys of
//     one head per lane) is P's operand layout for P V, so probabilities
//     never move;
//   * for P V each wave owns a block of output columns for all the
//     workgroup's heads and widens them from the raw tile with transposing
//     LDS reads (keys along the reduction axis), so no two waves hold partial
//     sums of one output and nothing is merged;
//   * online softmax in base 2 with lazy rescaling: the running maximum is
//     only raised when a tile's maximum exceeds it by more than 8 (so
//     probabilities stay below 2^8 in f16); the sink enters only the final
//     denominator.
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

constexpr int AT_HEADS = 16;
constexpr int AT_D = 512;
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

// x combined with the value of the lane 16 (32) away, in every lane: the
// gfx950 permlane swaps leave {x, x[lane ^ 16]} ({x, x[lane ^ 32]}) in the
// two results, with no LDS round trip
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
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

// LDS layout of a round's raw key bytes (row stride V3_RS) and of staged f16
// q rows (V3_QS); V3_SG scale groups per key at most (the pages' 288-byte
// records: one E4M3 scale per 16 dims).
constexpr int V3_RS = 528;
constexpr int V3_SG = 32;
constexpr int V3_QS = AT_D * 2 + 16;
// LDS byte offset of raw key row `row` of a round: every 16-row block is
// shifted by 8 bytes, so the transposing reads of two 16-lane groups (two
// different 16-row blocks at the same column) use disjoint banks.
__device__ __forceinline__ int v3_row(int row) { return row * V3_RS + (row >> 4) * 8; }
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

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

template <bool S16, bool TURN>
__global__ __launch_bounds__(64 * WD_WAVES) void sparse_attn_wide_kernel(AttnArgs a) {
  constexpr int NHB = 4;              // 16-head blocks
  constexpr int HW = 16 * NHB;        // heads per workgroup
  constexpr int CB = 4;               // 16-column blocks per wave
  __shared__ __attribute__((aligned(16))) uint8_t s_q[HW * V3_QS];
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[WD_RBUF];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[HW * WD_PS];
  __shared__ __attribute__((aligned(16))) _Float16 s_scl[V3_SG][WD_ROUND];
  __shared__ __attribute__((aligned(16))) float s_m[WD_WAVES][HW];

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // the workgroups of a query on one XCD (handed out round-robin)
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int n_hg = a.H / HW;
  const int split = bid % a.n_split;
  const int rest = bid / a.n_split;
  const int hg = rest % n_hg;
  const int t = rest / n_hg;
  const int h0 = hg * HW;

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
  // keys that do not exist are read from this query's own q rows (always
  // mapped, at least 16 KB) and get a zero scale and probability
  const uint8_t* dummy = (const uint8_t*)a.q + (int64_t)t * a.H * AT_D * 2;

  struct Raw {
    v4u d[8];
    float4 s;
    bool ok;
  };
  // the main-KV position of lane (r, g)'s key in round rd, -1 past the
  // workgroup's rounds (requested a round ahead, so the row loads never wait
  // on it).  The load is unconditional (a dummy address when there is no
  // key): a load under a branch makes every later wait count for the worst
  // path, and the round's first use of its rows then waited for this load too
  auto key_pos = [&](int rd) -> int {
    const int slot = (rd - n_swa_rounds) * WD_ROUND + 16 * wave + r;
    const bool has = rd < re && rd >= n_swa_rounds && slot < a.k;
    const int32_t* src = has ? irow + slot : (const int32_t*)dummy;
    const int v = *src;
    return has ? v : -1;
  };
  // lane (r, g): key r of the wave's 16, dims [128 g, +128)
  auto load_swa = [&](int rd, Raw& R) {
    const int slot = rd * WD_ROUND + 16 * wave + r;
    const int64_t row = sbase + min(slot, max(n_swa - 1, 0));   // past the window: the last row again
    const uint8_t* src = a.swa + row * a.swa_stride + 128 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) R.d[j] = *(const v4u*)(src + 16 * j);
    R.s = make_float4(a.swa_scale[row * a.swa_scale_stride + g], 0.f, 0.f, 0.f);
    R.ok = slot < n_swa;
  };
  // pos from key_pos
  auto load_main = [&](int pos, Raw& R) {
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
  };

  // ---- prologue
  Raw R;
  if (rb < re) {
    if (rb < n_swa_rounds) load_swa(rb, R);
    else load_main(key_pos(rb), R);
  }
  // positions of the next round's keys; each round requests those of the
  // round after next, so a position has a whole round to arrive before its
  // row is requested
  int pos_nx = key_pos(rb + 1);
  // q of all heads to LDS as f16
  {
    // thread i converts HW consecutive dims of head i / (512 / HW)
    constexpr int TPH = 64 * WD_WAVES / HW;   // threads per head
    const int qh = threadIdx.x / TPH, qd = (threadIdx.x % TPH) * HW;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t * a.H + h0 + qh) * AT_D + qd;
    v4u qraw[HW / 8];
#pragma unroll
    for (int c = 0; c < HW / 8; ++c) qraw[c] = *(const v4u*)(qrow + 8 * c);
#pragma unroll
    for (int c = 0; c < HW / 8; ++c) {
      v8h h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[2 * e] = (_Float16)__uint_as_float(qraw[c][e] << 16);
        h[2 * e + 1] = (_Float16)__uint_as_float(qraw[c][e] & 0xFFFF0000u);
      }
      *(v8h*)(s_q + qh * V3_QS + 2 * qd + 16 * c) = h;
    }
  }
  float sink2[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) sink2[hb] = a.sink[h0 + 16 * hb + r] * LOG2E;
  __syncthreads();   // s_q

  // O[hb][cb]: heads 16 hb + 4 g + j, column c0 + 16 cb + r
  v4f O[NHB][CB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[hb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_s[NHB], l_part[NHB];   // head 16 hb + r (log2 units); denominator over this wave's keys
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    m_s[hb] = -INFINITY;
    l_part[hb] = 0.f;
  }
  const float zscale = a.scale * LOG2E;
  const int c0 = wave * (16 * CB);
  const uint8_t* qsrc = s_q + r * V3_QS + 256 * g;

  // the B operands of step c of phase A (q of head block hb) come from LDS;
  // the reads of step c + 1 are issued before the products of step c (a
  // scheduling barrier keeps the compiler from sinking each read next to its
  // product, which left one LDS round trip exposed per product: 4,096-query
  // chunk, 622 -> 602 us per call)
  auto phase_a = [&](auto dequant_step, v4f (&acc)[NHB]) {
    {
      v8h qn[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        v8h qc[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) qc[hb] = qn[hb];
        if (c + 1 < 16) {
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) qn[hb] = *(const v8h*)(qsrc + 16 * hb * V3_QS + 16 * (c + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        const v8h kv = dequant_step(c);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qc[hb], acc[hb], 0, 0, 0);
      }
    }
  };

  // one round; SWA and main rounds are compiled apart so neither path keeps
  // the other's registers alive
  auto round = [&](auto swa_tag, int rd) {
    constexpr bool swa_round = decltype(swa_tag)::value;
    const int pos_nn = key_pos(rd + 2);
    // ---- phase A: S^T of the wave's 16 keys for the workgroup's heads
    v4f acc[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) acc[hb] = (v4f){0.f, 0.f, 0.f, 0.f};
    if constexpr (swa_round) {
      const float sc = R.s.x;
      const _Float16 mh = scale_mantissa(sc);
      const v2h m2 = {mh, mh};
      phase_a([&](int c) -> v8h {
        uint32_t kd[4];
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2], sc, m2, &kd[0]);
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2 + 1], sc, m2, &kd[2]);
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
        return __builtin_bit_cast(v8h, kv);
      }, acc);
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
      phase_a([&](int c) -> v8h {
        uint32_t kd[4];
        if (S16) {
          dequant_fp4x8_h(R.d[c >> 2][c & 3], s8[c >> 1], kd);
        } else {
          const _Float16 mh = scale_mantissa(s4[c >> 2]);
          dequant_fp4x8(R.d[c >> 2][c & 3], s4[c >> 2], (v2h){mh, mh}, kd);
        }
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
        return __builtin_bit_cast(v8h, kv);
      }, acc);
    }
    // lane (r, g) of S^T holds keys 4 g + i of the tile for head 16 hb + r
    const uint32_t ok4 = (uint32_t)(__ballot(R.ok) >> (4 * g)) & 0xFu;
    float z[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[hb][i] = ((ok4 >> i) & 1u) ? acc[hb][i] * zscale : -INFINITY;
      float mt = fmaxf(fmaxf(z[hb][0], z[hb][1]), fmaxf(z[hb][2], z[hb][3]));
      mt = max_xor32(max_xor16(mt));
      if (g == 0) s_m[wave][NHB * r + hb] = mt;
    }
    __syncthreads();

    // ---- phase B: running maxima (raised lazily, the same in every wave),
    // P, scales, raw bytes
    {
      bool raise = false;
      float alpha[NHB];
      // the maxima are stored [wave][r][head block]: one read of NHB floats per wave
      float mx[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) mx[hb] = s_m[0][NHB * r + hb];
#pragma unroll
      for (int w = 1; w < WD_WAVES; ++w)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) mx[hb] = fmaxf(mx[hb], s_m[w][NHB * r + hb]);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const bool up = mx[hb] > m_s[hb] + RESCALE_SLACK || (m_s[hb] == -INFINITY && mx[hb] > -INFINITY);
        const float m_new = up ? mx[hb] : m_s[hb];
        alpha[hb] = (m_new == -INFINITY || !up) ? 1.f : __builtin_amdgcn_exp2f(m_s[hb] - m_new);
        raise |= up;
        m_s[hb] = m_new;
        // z - m_new <= 8 here, and -inf gives 0 (also while no key of the
        // head has been seen: then every z is -inf and the reference is 0)
        const float mref = (m_new == -INFINITY) ? 0.f : m_new;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(z[hb][i] - mref);
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
        for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float aj = __shfl(alpha[hb], 4 * g + j);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) O[hb][cb][j] *= aj;
          }
        }
      }
    }
    __syncthreads();

    // ---- phase C: O[HW x 16 CB] += P (V * scale) over the round's keys
    auto phase_c = [&]() {
      const lds_u8* rawl = (const lds_u8*)s_raw;
      if constexpr (swa_round) {
        // 32-key blocks: lane group g holds keys 32 kb + 8 g .. + 7; the
        // wave's columns lie in one 128-dim scale group.  The column blocks'
        // V operands are widened first, then P streams by head block.
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int k0 = 32 * kb + 8 * g;
          const v8h S8 = *(const v8h*)(&s_scl[c0 >> 7][k0]);
          const int rrow = v3_row(k0 + (r >> 1));
          v8h B[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const v2i_t tv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + c0 + 16 * cb + 8 * (r & 1)));
            const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, false);
            const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, true);
            const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, false);
            const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, true);
            B[cb] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]} * S8;
          }
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            const v8h P = *(const v8h*)(s_p + (16 * hb + r) * WD_PS + 2 * k0);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, B[cb], O[hb][cb], 0, 0, 0);
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
          // block's P is read during the previous block's products (64 heads:
          // 602 -> 596 us per call on the same chunk)
          v8h B1[CB], B2[CB];
          v8h S1s[CB], S2s[CB];
          v2i_t tvs[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int grp = S16 ? ((c0 + 16 * cb) >> 4) : ((c0 + 16 * cb) >> 5);
            S1s[cb] = *(const v8h*)(&s_scl[grp][kt]);
            S2s[cb] = *(const v8h*)(&s_scl[grp][kt + 8]);
            tvs[cb] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + (c0 + 16 * cb) / 2));
          }
          v8h P1n = *(const v8h*)(s_p + r * WD_PS + 2 * kt);
          v8h P2n = *(const v8h*)(s_p + r * WD_PS + 2 * (kt + 8));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
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
          for (int hb = 0; hb < NHB; ++hb) {
            const v8h P1 = P1n, P2 = P2n;
            if (hb + 1 < NHB) {
              P1n = *(const v8h*)(s_p + (16 * (hb + 1) + r) * WD_PS + 2 * kt);
              P2n = *(const v8h*)(s_p + (16 * (hb + 1) + r) * WD_PS + 2 * (kt + 8));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
              O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P1, B1[cb], O[hb][cb], 0, 0, 0);
              O[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P2, B2[cb], O[hb][cb], 0, 0, 0);
            }
          }
        }
      }
    };
    // the next round's rows (this round's bytes are in LDS now), then phase
    // C.  Main rounds load unconditionally (after the last round: the dummy
    // row): with a branch around the loads the compiler waited ahead of phase
    // C for every load in flight, so no round overlapped its successor's
    // loads.  (SWA rounds keep that wait: a copy of phase C per load kind
    // raises the kernel past the register file.)
    const int pos = pos_nx;
    pos_nx = pos_nn;
    if constexpr (swa_round) {
      if (rd + 1 < n_swa_rounds) load_swa(rd + 1, R);
      else load_main(pos, R);
      phase_c();
    } else {
      load_main(pos, R);
      phase_c();
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
  for (int hb = 0; hb < NHB; ++hb) {
    float l = l_part[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (g == 0) s_m[wave][16 * hb + r] = l;
  }
  float* s_mx = (float*)s_p;   // [HW] running maxima, [HW] sink logits (log2 units)
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      s_mx[16 * hb + r] = m_s[hb];
      s_mx[HW + 16 * hb + r] = sink2[hb];
    }
  }
  __syncthreads();
  float Lh[NHB][4], Mh[NHB][4], Sk[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const v4f mv = *(const v4f*)(s_mx + 16 * hb + 4 * g);
    const v4f sv = *(const v4f*)(s_mx + HW + 16 * hb + 4 * g);
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
    for (int hb = 0; hb < NHB; ++hb) {
      float* rec = a.part + (((int64_t)t * (a.H / 16) + h0 / 16 + hb) * a.n_split + split) * ATTN_PART_FLOATS;
      if (wave == 0 && r == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rec[4 * g + j] = Mh[hb][j];
          rec[16 + 4 * g + j] = Lh[hb][j];
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) rec[32 + (4 * g + j) * AT_D + c0 + 16 * cb + r] = O[hb][cb][j];
    }
    return;
  }
  float fo[NHB][4];
  const bool write_lse = a.lse && wave == 0 && r == 0;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sk = Sk[hb][j];
      const float Mx = fmaxf(Mh[hb][j], sk);
      const float e_keys = (Mh[hb][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mh[hb][j] - Mx);
      const float den = Lh[hb][j] * e_keys + ((Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sk - Mx));
      fo[hb][j] = (den > 0.f) ? e_keys * __builtin_amdgcn_rcpf(den) : 0.f;
      if (write_lse) a.lse[(int64_t)t * a.H + h0 + 16 * hb + 4 * g + j] = (Mx + __builtin_amdgcn_logf(den)) * LN2;
    }
  // inverse RoPE of dims 448..511 (wave 7's columns): the pair (2i, 2i+1)
  // sits in lanes r, r ^ 1
  const bool turn = TURN && a.rope != nullptr && p >= 0 && p < a.n_rope && c0 >= 448;
  const float* csr = a.rope + (int64_t)max(p, 0) * 64;   // read only when turning
  // output through LDS (the raw tile is free), one 16-head block at a time:
  // each wave stages its 16 x 16 CB block, then every lane stores 16-byte runs
  constexpr int OSB = 16 * CB * 4 + 16;                  // staged row stride (bytes), room for fp32
  static_assert(WD_WAVES * 16 * OSB <= WD_RBUF, "the staged output fits the raw tile");
  uint8_t* ob = s_raw + wave * 16 * OSB;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      v4f v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = O[hb][cb][j] * fo[hb][j];
      if (TURN) {
        v4f vp;
#pragma unroll
        for (int j = 0; j < 4; ++j) vp[j] = __shfl_xor(v[j], 1);
        if (turn) {
          const int i = (c0 - 448 + 16 * cb + r) >> 1;
          const float c = csr[i], sn = csr[32 + i];
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
    // 16 rows of 16 CB fp32 columns: bf16 out in 8-column runs (hardware
    // round-to-nearest-even conversion); fp32 out in 4-column runs
    const int64_t orow = (int64_t)t * a.H + h0 + 16 * hb;
    if (a.out_bf16) {
      constexpr int LPR = 2 * CB;   // 16-byte runs per row
#pragma unroll
      for (int e0 = 0; e0 < 16 * LPR; e0 += 64) {
        const int e = e0 + lane;
        if (16 * LPR >= 64 || e < 16 * LPR) {
          const int row = e / LPR, ch = e % LPR;
          const v4f x0 = *(const v4f*)(ob + row * OSB + 32 * ch);
          const v4f x1 = *(const v4f*)(ob + row * OSB + 32 * ch + 16);
          v4u pk;
          pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[1]) << 16);
          pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[3]) << 16);
          pk[2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[1]) << 16);
          pk[3] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[3]) << 16);
          *(v4u*)((uint16_t*)a.out + (orow + row) * AT_D + c0 + 8 * ch) = pk;
        }
      }
    } else {
      constexpr int LPR = 4 * CB;   // 16-byte runs per row
#pragma unroll
      for (int e0 = 0; e0 < 16 * LPR; e0 += 64) {
        const int e = e0 + lane;
        const int row = e / LPR, ch = e % LPR;
        const v4u v = *(const v4u*)(ob + row * OSB + 16 * ch);
        *(v4u*)((float*)a.out + (orow + row) * AT_D + c0 + 4 * ch) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// Pipelined 16-head form: one workgroup = one query x 16 heads x one part of
// the output columns (x one key split), eight waves, rounds of 128 keys with
// one barrier per round.  A wave forms its tile's P against the tile's own
// per-head maximum m_t and publishes m_t and the tile's row sums; after the
// barrier every wave derives the same running maximum M from the tiles'
// maxima (raised lazily, by more than 8 only) and scales each tile's P by
// 2^(m_t - M) as it reads it for P V.  The LDS tiles (raw bytes, scales, P,
// tile statistics) are double-buffered, so one wave's phase A of round r + 1
// runs beside another's phase C of round r, and round r + 1's rows are
// requested as soon as round r's bytes are in LDS:
//
//   A  dequantize the wave's 16 keys in registers as the K operand of
//      S^T = K Q^T (q of the 16 heads in registers), put the raw bytes and
//      scales in the round's buffer, request the next round's rows, form and
//      store P and the tile statistics;
//   C  (after the barrier) running maximum, denominator, then P V for the
//      wave's 16 CB columns from transposing reads of the raw tile.
//
// A buffer written in phase A of round r + 2 was last read in phase C of
// round r, which every wave finishes before the barrier of round r + 1.
constexpr int PP_BUF = 2;

template <bool S16, bool TURN, int CB>
__global__ __launch_bounds__(64 * WD_WAVES) void sparse_attn_pipe_kernel(AttnArgs a) {
  constexpr int NCS = 4 / CB;         // column parts
  static_assert(CB == 1 || CB == 2 || CB == 4, "shape");
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[PP_BUF][WD_RBUF];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[PP_BUF][16 * WD_PS];
  __shared__ __attribute__((aligned(16))) _Float16 s_scl[PP_BUF][V3_SG][WD_ROUND];
  __shared__ __attribute__((aligned(16))) float s_st[PP_BUF][2][16][WD_WAVES];   // [m_t, l_t][head][tile]

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // the workgroups of a query on one XCD (handed out round-robin)
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int n_hg = a.H / 16;
  const int split = bid % a.n_split;
  int rest = bid / a.n_split;
  const int cs = rest % NCS;
  rest /= NCS;
  const int hg = rest % n_hg;
  const int t = rest / n_hg;
  const int h0 = hg * 16;

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
  // keys that do not exist are read from this query's own q rows (always
  // mapped, at least 16 KB) and get a zero scale and probability
  const uint8_t* dummy = (const uint8_t*)a.q + (int64_t)t * a.H * AT_D * 2;

  struct Raw {
    v4u d[8];
    float4 s;
    bool ok;
  };
  // the main-KV position of lane (r, g)'s key in round rd, -1 past the
  // workgroup's rounds; the load is unconditional (a dummy address when
  // there is no key), as a load under a branch makes later waits count for
  // the worst path
  auto key_pos = [&](int rd) -> int {
    const int slot = (rd - n_swa_rounds) * WD_ROUND + 16 * wave + r;
    const bool has = rd < re && rd >= n_swa_rounds && slot < a.k;
    const int32_t* src = has ? irow + slot : (const int32_t*)dummy;
    const int v = *src;
    return has ? v : -1;
  };
  // lane (r, g): key r of the wave's 16, dims [128 g, +128)
  auto load_swa = [&](int rd, Raw& R) {
    const int slot = rd * WD_ROUND + 16 * wave + r;
    const int64_t row = sbase + min(slot, max(n_swa - 1, 0));   // past the window: the last row again
    const uint8_t* src = a.swa + row * a.swa_stride + 128 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) R.d[j] = *(const v4u*)(src + 16 * j);
    R.s = make_float4(a.swa_scale[row * a.swa_scale_stride + g], 0.f, 0.f, 0.f);
    R.ok = slot < n_swa;
  };
  auto load_main = [&](int pos, Raw& R) {
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
  };

  // ---- prologue
  Raw R;
  if (rb < re) {
    if (rb < n_swa_rounds) load_swa(rb, R);
    else load_main(key_pos(rb), R);
  }
  // positions of the next round's keys; each round requests those of the
  // round after next, so a position has a whole round to arrive
  int pos_nx = key_pos(rb + 1);
  // q of the 16 heads as f16, staged through buffer 1's raw tile (first
  // written in round rb + 1, after every wave has passed round rb's barrier):
  // each thread converts 16 dims, then every wave reads its B operands, lane
  // (r, g) head h0 + r, dims 128 g + 8 c .. + 7 for step c
  {
    const int qh = threadIdx.x >> 5, qd = (threadIdx.x & 31) * 16;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t * a.H + h0 + qh) * AT_D + qd;
    const v4u q0 = *(const v4u*)qrow, q1 = *(const v4u*)(qrow + 8);
    v8h h0v, h1v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h0v[2 * e] = (_Float16)__uint_as_float(q0[e] << 16);
      h0v[2 * e + 1] = (_Float16)__uint_as_float(q0[e] & 0xFFFF0000u);
      h1v[2 * e] = (_Float16)__uint_as_float(q1[e] << 16);
      h1v[2 * e + 1] = (_Float16)__uint_as_float(q1[e] & 0xFFFF0000u);
    }
    *(v8h*)(s_raw[1] + qh * V3_QS + 2 * qd) = h0v;
    *(v8h*)(s_raw[1] + qh * V3_QS + 2 * qd + 16) = h1v;
  }
  __syncthreads();
  v8h qreg[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qreg[c] = *(const v8h*)(s_raw[1] + r * V3_QS + 256 * g + 16 * c);

  // O[cb]: heads 4 g + j, column c0 + 16 cb + r
  v4f O[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) O[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY;   // running maximum of head r (log2 units), the same in every wave
  float L = 0.f;         // denominator of head r relative to M
  const float zscale = a.scale * LOG2E;
  const int c0 = cs * (128 * CB) + wave * (16 * CB);

  auto round = [&](auto swa_tag, int rd) {
    constexpr bool swa_round = decltype(swa_tag)::value;
    const int bf = (rd - rb) & 1;
    const int pos_nn = key_pos(rd + 2);
    // ---- phase A: S^T of the wave's 16 keys for the 16 heads
    v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
    if constexpr (swa_round) {
      const float sc = R.s.x;
      const _Float16 mh = scale_mantissa(sc);
      const v2h m2 = {mh, mh};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        uint32_t kd[4];
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2], sc, m2, &kd[0]);
        dequant_fp8x4(R.d[c >> 1][(c & 1) * 2 + 1], sc, m2, &kd[2]);
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qreg[c], acc, 0, 0, 0);
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
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        uint32_t kd[4];
        if (S16) {
          dequant_fp4x8_h(R.d[c >> 2][c & 3], s8[c >> 1], kd);
        } else {
          const _Float16 mh = scale_mantissa(s4[c >> 2]);
          dequant_fp4x8(R.d[c >> 2][c & 3], s4[c >> 2], (v2h){mh, mh}, kd);
        }
        const v4u kv = {kd[0], kd[1], kd[2], kd[3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kv), qreg[c], acc, 0, 0, 0);
      }
    }
    // the round's raw bytes and scales (f16, zero for keys that do not exist)
    // to LDS, then the next round's rows into the freed registers
    const bool ok = R.ok;
    {
      const float4 cs4 = ok ? R.s : make_float4(0.f, 0.f, 0.f, 0.f);
      const int key = 16 * wave + r;
      uint8_t* dst = s_raw[bf] + v3_row(key);
      if constexpr (swa_round) {
        s_scl[bf][g][key] = (_Float16)cs4.x;
#pragma unroll
        for (int j = 0; j < 8; ++j) *(v4u*)(dst + 128 * g + 16 * j) = R.d[j];
      } else {
        if (S16) {
          const uint32_t w0 = __float_as_uint(cs4.x), w1 = __float_as_uint(cs4.y);
          const v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
          const v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
          const v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
          const v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
          s_scl[bf][8 * g + 0][key] = a0[0];
          s_scl[bf][8 * g + 1][key] = a0[1];
          s_scl[bf][8 * g + 2][key] = a1[0];
          s_scl[bf][8 * g + 3][key] = a1[1];
          s_scl[bf][8 * g + 4][key] = a2[0];
          s_scl[bf][8 * g + 5][key] = a2[1];
          s_scl[bf][8 * g + 6][key] = a3[0];
          s_scl[bf][8 * g + 7][key] = a3[1];
        } else {
          s_scl[bf][4 * g + 0][key] = (_Float16)cs4.x;
          s_scl[bf][4 * g + 1][key] = (_Float16)cs4.y;
          s_scl[bf][4 * g + 2][key] = (_Float16)cs4.z;
          s_scl[bf][4 * g + 3][key] = (_Float16)cs4.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *(v4u*)(dst + 64 * g + 16 * j) = R.d[j];
      }
    }
    const int pos = pos_nx;
    pos_nx = pos_nn;
    if constexpr (swa_round) {
      if (rd + 1 < n_swa_rounds) load_swa(rd + 1, R);
      else load_main(pos, R);
    } else {
      load_main(pos, R);
    }
    // tile statistics: lane (r, g) of S^T holds keys 4 g + i for head r
    {
      // validity of keys 4 g .. 4 g + 3 (lanes 4 g + i hold them)
      const uint32_t ok4 = (uint32_t)(__ballot(ok) >> (4 * g)) & 0xFu;
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = ((ok4 >> i) & 1u) ? acc[i] * zscale : -INFINITY;
      float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mt = max_xor32(max_xor16(mt));
      const float mref = (mt == -INFINITY) ? 0.f : mt;   // no key: every z is -inf, P is 0
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(z[i] - mref);
      float lt = (pv[0] + pv[1]) + (pv[2] + pv[3]);
      lt = add_xor32(add_xor16(lt));
      const v4h P4 = {(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
      *(v4h*)(s_p[bf] + r * WD_PS + 2 * (16 * wave + 4 * g)) = P4;
      if (g == 0) {
        s_st[bf][0][r][wave] = mt;
        s_st[bf][1][r][wave] = lt;
      }
    }
    __syncthreads();

    // ---- phase C: running maximum, denominator, O[16 x 16 CB] += P V
    // SWA rounds: 2^(m_t - M) of every tile for head r; main rounds (whose
    // products take tiles g and 4 + g in lane group g): only those two, the
    // maximum and the denominator's sum combined across the lane groups
    float f[WD_WAVES];
    float f_g[2];
    {
      float mt[WD_WAVES], lt[WD_WAVES], mx;
      if constexpr (swa_round) {
        const v4f ma = *(const v4f*)(&s_st[bf][0][r][0]), mb = *(const v4f*)(&s_st[bf][0][r][4]);
        const v4f la = *(const v4f*)(&s_st[bf][1][r][0]), lb = *(const v4f*)(&s_st[bf][1][r][4]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          mt[w] = ma[w];
          mt[4 + w] = mb[w];
          lt[w] = la[w];
          lt[4 + w] = lb[w];
        }
        mx = mt[0];
#pragma unroll
        for (int w = 1; w < WD_WAVES; ++w) mx = fmaxf(mx, mt[w]);
      } else {
        mt[0] = s_st[bf][0][r][g];
        mt[1] = s_st[bf][0][r][4 + g];
        lt[0] = s_st[bf][1][r][g];
        lt[1] = s_st[bf][1][r][4 + g];
        mx = max_xor32(max_xor16(fmaxf(mt[0], mt[1])));
      }
      const bool up = mx > M + RESCALE_SLACK || (M == -INFINITY && mx > -INFINITY);
      const float m_new = up ? mx : M;
      const float alpha = (m_new == -INFINITY || !up) ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
      M = m_new;
      const float mref = (M == -INFINITY) ? 0.f : M;
      float add = 0.f;
      // m_t - M <= 8 here, and -inf gives 0
      if constexpr (swa_round) {
#pragma unroll
        for (int w = 0; w < WD_WAVES; ++w) {
          f[w] = __builtin_amdgcn_exp2f(mt[w] - mref);
          add += f[w] * lt[w];
        }
      } else {
        f_g[0] = __builtin_amdgcn_exp2f(mt[0] - mref);
        f_g[1] = __builtin_amdgcn_exp2f(mt[1] - mref);
        add = add_xor32(add_xor16(f_g[0] * lt[0] + f_g[1] * lt[1]));
      }
      L = L * alpha + add;
      // every wave takes the same decision (same maxima, same rule)
      if (__any(up)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * g + j);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) O[cb][j] *= aj;
        }
      }
    }
    {
      const lds_u8* rawl = (const lds_u8*)s_raw[bf];
      const uint8_t* pb = s_p[bf] + r * WD_PS;
      if constexpr (swa_round) {
        // 32-key blocks: lane group g holds keys 32 kb + 8 g .. + 7 (tile
        // 2 kb + g / 2); the wave's columns lie in one 128-dim scale group
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int k0 = 32 * kb + 8 * g;
          const v8h S8 = *(const v8h*)(&s_scl[bf][c0 >> 7][k0]);
          const int rrow = v3_row(k0 + (r >> 1));
          // the keys' scales (one 128-dim group for all the wave's
          // columns) go into P, so V is the exact widened codes
          v8h B[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const v2i_t tv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + c0 + 16 * cb + 8 * (r & 1)));
            const v2h x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, false);
            const v2h x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[0], 1.0f, true);
            const v2h x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, false);
            const v2h x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)tv[1], 1.0f, true);
            B[cb] = (v8h){x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
          }
          const _Float16 fT = (_Float16)((g >> 1) ? f[2 * kb + 1] : f[2 * kb]);
          const v8h P = (*(const v8h*)(pb + 2 * k0) * (v8h){fT, fT, fT, fT, fT, fT, fT, fT}) * S8;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, B[cb], O[cb], 0, 0, 0);
        }
      } else {
        // halves of 64 keys: lane group g holds tile 4 half + g (16 keys);
        // one transposing read gives those 16 keys of one column (keys 0..7
        // and 8..15 feed two products).  Every LDS read of the half is
        // issued before the conversions.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 16 * (4 * half + g);
          const int rrow = v3_row(kt + r);
          v8h S1s[CB], S2s[CB];
          v2i_t tvs[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int grp = S16 ? ((c0 + 16 * cb) >> 4) : ((c0 + 16 * cb) >> 5);
            S1s[cb] = *(const v8h*)(&s_scl[bf][grp][kt]);
            S2s[cb] = *(const v8h*)(&s_scl[bf][grp][kt + 8]);
            tvs[cb] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(rawl + rrow + (c0 + 16 * cb) / 2));
          }
          const v8h P1r = *(const v8h*)(pb + 2 * kt);
          const v8h P2r = *(const v8h*)(pb + 2 * (kt + 8));
          __builtin_amdgcn_sched_barrier(0);
          const _Float16 fT = (_Float16)f_g[half];
          const v8h f8 = {fT, fT, fT, fT, fT, fT, fT, fT};
          const v8h P1 = P1r * f8, P2 = P2r * f8;
          // with one scale per 32 dims the wave's columns span NG scale
          // groups (CB = 4: two); their scales go into P, once per group,
          // instead of into every column block's V
          constexpr int NG = S16 ? 1 : (CB == 4 ? 2 : 1);
          v8h P1g[NG], P2g[NG];
          if (!S16) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
              P1g[gi] = P1 * S1s[2 * gi];
              P2g[gi] = P2 * S2s[2 * gi];
            }
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
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
            if (S16) {
              const v8h B1 = __builtin_bit_cast(v8h, u1) * S1s[cb];
              const v8h B2 = __builtin_bit_cast(v8h, u2) * S2s[cb];
              O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P1, B1, O[cb], 0, 0, 0);
              O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P2, B2, O[cb], 0, 0, 0);
            } else {
              const int gi = (CB == 4) ? (cb >> 1) : 0;
              O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P1g[gi], __builtin_bit_cast(v8h, u1), O[cb], 0, 0, 0);
              O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P2g[gi], __builtin_bit_cast(v8h, u2), O[cb], 0, 0, 0);
            }
          }
        }
      }
    }
  };
  int rd = rb;
  for (; rd < min(re, n_swa_rounds); ++rd) round(std::true_type{}, rd);
  for (; rd < re; ++rd) round(std::false_type{}, rd);

  // ---- epilogue: M and L of head r are the same in every wave; wave 0
  // publishes them with the sink, and each lane takes its O rows' values
  __syncthreads();   // every wave is past its last read of the buffers
  float* s_ml = (float*)s_p[0];   // [16] M, [16] L, [16] sink logits (log2 units)
  if (wave == 0 && g == 0) {
    s_ml[r] = M;
    s_ml[16 + r] = L;
    s_ml[32 + r] = a.sink[h0 + r] * LOG2E;
  }
  __syncthreads();
  const v4f Mv = *(const v4f*)(s_ml + 4 * g);
  const v4f Lv = *(const v4f*)(s_ml + 16 + 4 * g);
  const v4f Sv = *(const v4f*)(s_ml + 32 + 4 * g);
  if (a.n_split > 1) {
    // partial record of the 16 heads (the layout the combine reads): per
    // head the running maximum (log2 units, no sink), the denominator and O,
    // all relative to that maximum; each column part writes its columns
    float* rec = a.part + (((int64_t)t * n_hg + hg) * a.n_split + split) * ATTN_PART_FLOATS;
    if (wave == 0 && r == 0 && cs == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rec[4 * g + j] = Mv[j];
        rec[16 + 4 * g + j] = Lv[j];
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) rec[32 + (4 * g + j) * AT_D + c0 + 16 * cb + r] = O[cb][j];
    return;
  }
  float fo[4];
  const bool write_lse = a.lse && wave == 0 && r == 0 && cs == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sk = Sv[j];
    const float Mx = fmaxf(Mv[j], sk);
    const float e_keys = (Mv[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mv[j] - Mx);
    const float den = Lv[j] * e_keys + ((Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sk - Mx));
    fo[j] = (den > 0.f) ? e_keys * __builtin_amdgcn_rcpf(den) : 0.f;
    if (write_lse) a.lse[(int64_t)t * a.H + h0 + 4 * g + j] = (Mx + __builtin_amdgcn_logf(den)) * LN2;
  }
  // inverse RoPE of dims 448..511 (the waves whose columns lie there): the
  // pair (2i, 2i+1) sits in lanes r, r ^ 1
  const bool turn = TURN && a.rope != nullptr && p >= 0 && p < a.n_rope && c0 >= 448;
  const float* csr = a.rope + (int64_t)max(p, 0) * 64;   // read only when turning
  // output through LDS (the raw tiles are free): each wave stages its
  // 16 x 16 CB block, then every lane stores 16-byte runs
  constexpr int OSB = 16 * CB * 4 + 16;                  // staged row stride (bytes), room for fp32
  static_assert(WD_WAVES * 16 * OSB <= WD_RBUF, "the staged output fits a raw tile");
  uint8_t* ob = s_raw[0] + wave * 16 * OSB;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    v4f v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = O[cb][j] * fo[j];
    if (TURN) {
      v4f vp;
#pragma unroll
      for (int j = 0; j < 4; ++j) vp[j] = __shfl_xor(v[j], 1);
      if (turn) {
        const int i = (c0 - 448 + 16 * cb + r) >> 1;
        const float c = csr[i], sn = csr[32 + i];
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
  // 16 rows of 16 CB fp32 columns: bf16 out in 8-column runs (hardware
  // round-to-nearest-even conversion); fp32 out in 4-column runs
  const int64_t orow = (int64_t)t * a.H + h0;
  if (a.out_bf16) {
    constexpr int LPR = 2 * CB;   // 16-byte runs per row
#pragma unroll
    for (int e0 = 0; e0 < 16 * LPR; e0 += 64) {
      const int e = e0 + lane;
      if (16 * LPR >= 64 || e < 16 * LPR) {
        const int row = e / LPR, ch = e % LPR;
        const v4f x0 = *(const v4f*)(ob + row * OSB + 32 * ch);
        const v4f x1 = *(const v4f*)(ob + row * OSB + 32 * ch + 16);
        v4u pk;
        pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[1]) << 16);
        pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0[3]) << 16);
        pk[2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[1]) << 16);
        pk[3] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1[3]) << 16);
        *(v4u*)((uint16_t*)a.out + (orow + row) * AT_D + c0 + 8 * ch) = pk;
      }
    }
  } else {
    constexpr int LPR = 4 * CB;   // 16-byte runs per row
#pragma unroll
    for (int e0 = 0; e0 < 16 * LPR; e0 += 64) {
      const int e = e0 + lane;
      const int row = e / LPR, ch = e % LPR;
      const v4u v = *(const v4u*)(ob + row * OSB + 16 * ch);
      *(v4u*)((float*)a.out + (orow + row) * AT_D + c0 + 4 * ch) = v;
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

// Launch shape of the quantized path: the 64-head kernel (nhb 4: one
// workgroup per query and 64 heads) or the pipelined 16-head kernel with cb
// 16-column blocks per wave (4 / cb column parts), and ns key splits.
struct AttnPlan {
  int nhb, cb, ns;
};

static int ceil_div(int x, int y) { return (x + y - 1) / y; }

static AttnPlan attn_plan(int Q, int H, int k, int window) {
  AttnPlan pl = {1, 4, 1};
  if (Q <= 0) return pl;
  if (H % 64 == 0 && Q * (H / 64) >= 256) {
    pl.nhb = 4;   // one workgroup per query and 64 heads fills the chip
    return pl;
  }
  // 16-head groups; with fewer than the chip's 256 CUs the columns are
  // parted (each part recomputes the scores, but nothing is merged and the
  // rows come from L2), and below 128 workgroups the keys are split as well
  // (partial records cost as many bytes as the rows they summarise)
  const int groups = Q * (H / 16);
  if (groups >= 256) return pl;
  pl.cb = groups >= 128 ? 2 : 1;
  const int wgs = groups * (4 / pl.cb);
  const int rounds = ceil_div(window, WD_ROUND) + ceil_div(k, WD_ROUND);
  if (wgs < 128) pl.ns = max(1, min(min(rounds, ATTN_MAX_SPLIT), ceil_div(128, wgs)));
  return pl;
}

// Key splits per (query, 16 heads) the launch will use when the caller
// passes the workspace.
int attn_splits(int Q, int H, int k, int window) { return attn_plan(Q, H, k, window).ns; }

template <bool S16, bool TURN>
static void launch_wide_n(const AttnArgs& a, hipStream_t s) {
  const int wgs = a.Q * (a.H / 64) * a.n_split;
  hipLaunchKernelGGL((sparse_attn_wide_kernel<S16, TURN>), dim3(wgs), dim3(64 * WD_WAVES), 0, s, a);
}

template <bool S16, bool TURN, int CB>
static void launch_pipe_n(const AttnArgs& a, hipStream_t s) {
  const int wgs = a.Q * (a.H / 16) * (4 / CB) * a.n_split;
  hipLaunchKernelGGL((sparse_attn_pipe_kernel<S16, TURN, CB>), dim3(wgs), dim3(64 * WD_WAVES), 0, s, a);
}

template <bool S16, bool TURN>
static hipError_t launch_attn(const AttnArgs& a, const AttnPlan& pl, hipStream_t s) {
  switch (pl.nhb * 10 + pl.cb) {
    case 44: launch_wide_n<S16, TURN>(a, s); break;
    case 14: launch_pipe_n<S16, TURN, 4>(a, s); break;
    case 12: launch_pipe_n<S16, TURN, 2>(a, s); break;
    case 11: launch_pipe_n<S16, TURN, 1>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn_quant(const AttnArgs& a, hipStream_t s) {
  const int groups = a.Q * (a.H / AT_HEADS);
  const AttnPlan pl = attn_plan(a.Q, a.H, a.k, a.window);
  // split calls turn the output in the combine kernel
  const bool turn = a.rope != nullptr && a.n_split == 1;
  const hipError_t e = a.main_s16 ? (turn ? launch_attn<true, true>(a, pl, s) : launch_attn<true, false>(a, pl, s))
                                  : (turn ? launch_attn<false, true>(a, pl, s) : launch_attn<false, false>(a, pl, s));
  if (e != hipSuccess) return e;
  if (a.n_split > 1) launch_combine(a, groups, s);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_attn_f32_kernel, dim3(a.Q * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
