// Top-k selection and block-candidate selection for the CSA2 hot path.
//
// Both calls choose, per row, the k best entries under the strict order
// (value descending, position ascending) among entries whose value is above
// -inf, and emit the chosen positions ascending, padded with -1 (DSA page,
// "Top-k: tokens, not blocks"; CSA2 page, "hierarchical sparse indexer" and
// "where attention is computed" for the block pool with the latest block
// forced).
//
// One workgroup of 1024 threads selects within a chunk of up to 32768
// entries held in LDS as order-preserving 32-bit keys:
//   1. load the chunk (dense scores, pool scores, block maxima of 8-score
//      blocks, or a (key, position) list from a previous stage);
//   2. if more than k entries are selectable, radix-select the k-th largest
//      key T with four 8-bit digit passes over LDS histograms;
//   3. compact in position order with wave ballots: every key > T, then the
//      first (k - #greater) keys equal to T, which applies the lower-position
//      tie rule exactly.
// Long rows are cut into chunks; each chunk's k winners (already in position
// order) form a shorter list, and further stages select from the lists until
// one chunk holds the row.  A strict total order makes this exact: an entry
// among the row's k best is among its chunk's k best.
#include "kernels.h"

namespace csa2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;  // key of -inf: selectable keys are larger
constexpr uint32_t KEY_POS_INF = 0xFF800000u;  // key of +inf (the forced latest block)
constexpr uint32_t KEY_PAD = 0u;               // padding in candidate lists

__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct StageArgs {
  SelectArgs s;
  const uint32_t* in_key;
  const int32_t* in_pos;
  int64_t in_len;        // list length per row (LIST mode)
  int chunk;             // entries per chunk
  uint32_t* out_key;     // list output, [Q][out_stride]; null for the final stage
  int32_t* out_pos;
  int64_t out_stride;
};

__device__ __forceinline__ int sel_visible(const SelectArgs& s, int t) {
  return (int)(((int64_t)s.q_pos[t] + 1) / s.ratio);
}

template <int MODE>
__device__ __forceinline__ int64_t row_length(const StageArgs& a, int t) {
  const SelectArgs& s = a.s;
  if (MODE == SEL_DENSE) return s.q_pos ? min(s.n_cols, sel_visible(s, t)) : s.n_cols;
  if (MODE == SEL_POOL) return s.n_cols;
  if (MODE == SEL_BLOCKMAX) {
    const int n = min(s.n_cols, sel_visible(s, t));
    return n <= 0 ? 0 : ((n - 1) >> s.block_shift) + 1;
  }
  return a.in_len;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}

template <int MODE, int CAP>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(StageArgs a) {
  __shared__ uint32_t s_key[CAP];
  __shared__ int32_t s_pos[MODE == SEL_LIST ? CAP : 1];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_wsum[SEL_WAVES];
  __shared__ uint32_t s_gt[SEL_WAVES], s_eq[SEL_WAVES];
  __shared__ uint32_t s_bucket, s_above, s_nsel;

  const SelectArgs& s = a.s;
  const int t = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int64_t L = row_length<MODE>(a, t);
  const int64_t g0 = (int64_t)c * a.chunk;
  const int count = (int)max((int64_t)0, min((int64_t)a.chunk, L - g0));
  const float* row = s.scores + (int64_t)t * s.score_stride;

  if (tid == 0) s_nsel = 0;
  __syncthreads();

  // 1. load keys ------------------------------------------------------------
  uint32_t my_sel = 0;
  for (int i = tid; i < count; i += SEL_THREADS) {
    const int64_t g = g0 + i;
    uint32_t key;
    if (MODE == SEL_DENSE) {
      key = float_key(row[g]);
    } else if (MODE == SEL_POOL) {
      const int cb = s.cand[(int64_t)t * s.n_cand_blocks + (int)(g >> s.block_shift)];
      key = cb >= 0 ? float_key(row[g]) : KEY_NEG_INF;
    } else if (MODE == SEL_BLOCKMAX) {
      const int n = min(s.n_cols, sel_visible(s, t));
      const int p0 = (int)(g << s.block_shift);
      const int p1 = min(n, p0 + (1 << s.block_shift));
      float m = -INFINITY;
      for (int p = p0; p < p1; ++p) m = fmaxf(m, row[p]);
      key = (g == L - 1) ? KEY_POS_INF : float_key(m);
    } else {
      key = a.in_key[(int64_t)t * a.in_len + g];
      s_pos[i] = a.in_pos[(int64_t)t * a.in_len + g];
    }
    s_key[i] = key;
    my_sel += key > KEY_NEG_INF;
  }
  // block-wide count of selectable entries
  for (int d = 32; d >= 1; d >>= 1) my_sel += __shfl_xor(my_sel, d);
  if (lane == 0) atomicAdd(&s_nsel, my_sel);
  __syncthreads();
  const uint32_t nsel = s_nsel;
  const int k = s.k;

  // 2. radix select of the k-th largest key ---------------------------------
  uint32_t T, keq;
  if (nsel <= (uint32_t)k) {
    T = KEY_NEG_INF;
    keq = 0;
  } else {
    uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) s_hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < count; i += SEL_THREADS) {
        const uint32_t key = s_key[i];
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // suffix counts over buckets, highest bucket first
      const uint32_t cnt = (tid < 256) ? s_hist[255 - tid] : 0u;
      uint32_t incl = wave_incl_scan(cnt, lane);
      if (lane == 63) s_wsum[wave] = incl;
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < wave; ++w) incl += s_wsum[w];
        const uint32_t excl = incl - cnt;
        if (excl < krem && incl >= krem) {
          s_bucket = 255u - (uint32_t)tid;
          s_above = excl;
        }
      }
      __syncthreads();
      krem -= s_above;
      prefix |= s_bucket << shift;
      mask |= 255u << shift;
    }
    T = prefix;
    keq = krem;
  }

  // 3. order-preserving compaction ------------------------------------------
  const int seg = ((count + SEL_WAVES - 1) / SEL_WAVES + 63) & ~63;
  const int sb = min(count, wave * seg);
  const int se = min(count, sb + seg);
  uint32_t ngt = 0, neq = 0;
  for (int i0 = sb; i0 < se; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t key = (i < se) ? s_key[i] : KEY_PAD;
    ngt += __popcll(__ballot(key > T));
    neq += __popcll(__ballot(i < se && key == T));
  }
  if (lane == 0) {
    s_gt[wave] = ngt;
    s_eq[wave] = neq;
  }
  __syncthreads();
  // equal keys are taken in position order: wave w takes
  // min(eq_w, keq - (equal keys in earlier waves)) of them
  uint32_t cum_eq = 0, sel_before = 0, total = 0, run_eq = 0;
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t take_eq = min(s_eq[w], keq > cum_eq ? keq - cum_eq : 0u);
    const uint32_t selw = s_gt[w] + take_eq;
    if (w < wave) {
      sel_before += selw;
      run_eq += s_eq[w];
    }
    total += selw;
    cum_eq += s_eq[w];
  }
  uint32_t run_sel = sel_before;
  for (int i0 = sb; i0 < se; i0 += 64) {
    const int i = i0 + lane;
    const bool in = i < se;
    const uint32_t key = in ? s_key[i] : KEY_PAD;
    const bool is_gt = key > T;
    const bool is_eq = in && key == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t eq_rank = run_eq + lanes_below(eqm, lane);
    const bool take = is_gt || (is_eq && eq_rank < keq);
    const uint64_t selm = __ballot(take);
    if (take) {
      const uint32_t o = run_sel + lanes_below(selm, lane);
      const int64_t g = g0 + i;
      int32_t pos;
      if (MODE == SEL_DENSE || MODE == SEL_BLOCKMAX) {
        pos = (int32_t)g;
      } else if (MODE == SEL_POOL) {
        const int cb = s.cand[(int64_t)t * s.n_cand_blocks + (int)(g >> s.block_shift)];
        pos = (cb << s.block_shift) | (int)(g & ((1 << s.block_shift) - 1));
      } else {
        pos = s_pos[i];
      }
      if (a.out_key) {
        const int64_t off = (int64_t)t * a.out_stride + (int64_t)c * k + o;
        a.out_key[off] = key;
        a.out_pos[off] = pos;
      } else {
        s.out_idx[(int64_t)t * k + o] = pos;
      }
    }
    run_eq += __popcll(eqm);
    run_sel += __popcll(selm);
  }
  // padding
  for (int o = (int)total + tid; o < k; o += SEL_THREADS) {
    if (a.out_key) {
      const int64_t off = (int64_t)t * a.out_stride + (int64_t)c * k + o;
      a.out_key[off] = KEY_PAD;
      a.out_pos[off] = -1;
    } else {
      s.out_idx[(int64_t)t * k + o] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// host-side planning

static int pow2_ceil(int64_t x) {
  int p = 1;
  while (p < x && p < (1 << 30)) p <<= 1;
  return p;
}

SelectPlan plan_select(int Q, int64_t rows_len, int k) {
  SelectPlan p = {};
  if (rows_len <= SEL_CAP) {
    p.n_stages = 1;
    p.chunk1 = SEL_CAP;
    p.n_chunks1 = 1;
    p.ws_list_max = 0;
    return p;
  }
  // first stage: enough workgroups to spread the row over the chip, and a
  // reduction of at least 4x per chunk
  int c1 = pow2_ceil((rows_len * (int64_t)Q + 255) / 256);
  c1 = max(c1, pow2_ceil(4 * (int64_t)k));
  c1 = min(c1, SEL_CAP);
  p.chunk1 = c1;
  p.n_chunks1 = (int)((rows_len + c1 - 1) / c1);
  int64_t len = (int64_t)p.n_chunks1 * k;
  int st = 0;
  p.list_len[st++] = len;
  p.ws_list_max = len;
  while (len > SEL_CAP_LIST && st < 7) {
    const int64_t nch = (len + SEL_CAP_LIST - 1) / SEL_CAP_LIST;
    len = nch * k;
    p.list_len[st++] = len;
  }
  p.n_stages = st + 1;
  return p;
}

size_t select_workspace_bytes(int Q, int64_t rows_len, int k) {
  const SelectPlan p = plan_select(Q, rows_len, k);
  if (p.n_stages == 1) return 0;
  // two ping-pong lists of (key, position) pairs
  return (size_t)2 * (size_t)Q * (size_t)p.ws_list_max * 8u;
}

template <int MODE>
static hipError_t launch_first(const StageArgs& a, int nchunks, int Q, hipStream_t s) {
  hipLaunchKernelGGL((select_kernel<MODE, SEL_CAP>), dim3(nchunks, Q), dim3(SEL_THREADS), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_select(int mode, const SelectArgs& sa, int64_t rows_len, hipStream_t s) {
  const SelectPlan p = plan_select(sa.Q, rows_len, sa.k);
  StageArgs a = {};
  a.s = sa;
  if (p.n_stages == 1) {
    a.chunk = SEL_CAP;
    a.out_key = nullptr;
    switch (mode) {
      case SEL_DENSE: return launch_first<SEL_DENSE>(a, 1, sa.Q, s);
      case SEL_POOL: return launch_first<SEL_POOL>(a, 1, sa.Q, s);
      default: return launch_first<SEL_BLOCKMAX>(a, 1, sa.Q, s);
    }
  }
  uint8_t* ws = (uint8_t*)sa.workspace;
  const size_t list_bytes = (size_t)sa.Q * (size_t)p.ws_list_max * 4u;
  uint32_t* key_buf[2] = {(uint32_t*)ws, (uint32_t*)(ws + 2 * list_bytes)};
  int32_t* pos_buf[2] = {(int32_t*)(ws + list_bytes), (int32_t*)(ws + 3 * list_bytes)};

  // stage 1: from scores into list 0
  a.chunk = p.chunk1;
  a.out_key = key_buf[0];
  a.out_pos = pos_buf[0];
  a.out_stride = p.list_len[0];
  hipError_t e;
  switch (mode) {
    case SEL_DENSE: e = launch_first<SEL_DENSE>(a, p.n_chunks1, sa.Q, s); break;
    case SEL_POOL: e = launch_first<SEL_POOL>(a, p.n_chunks1, sa.Q, s); break;
    default: e = launch_first<SEL_BLOCKMAX>(a, p.n_chunks1, sa.Q, s); break;
  }
  if (e != hipSuccess) return e;
  // list stages
  int cur = 0;
  for (int st = 1; st < p.n_stages; ++st) {
    StageArgs b = {};
    b.s = sa;
    b.in_key = key_buf[cur];
    b.in_pos = pos_buf[cur];
    b.in_len = p.list_len[st - 1];
    const bool last = (st == p.n_stages - 1);
    int nch;
    if (last) {
      b.chunk = SEL_CAP_LIST;
      b.out_key = nullptr;
      nch = 1;
    } else {
      b.chunk = SEL_CAP_LIST;
      b.out_key = key_buf[cur ^ 1];
      b.out_pos = pos_buf[cur ^ 1];
      b.out_stride = p.list_len[st];
      nch = (int)((b.in_len + SEL_CAP_LIST - 1) / SEL_CAP_LIST);
    }
    hipLaunchKernelGGL((select_kernel<SEL_LIST, SEL_CAP_LIST>), dim3(nch, sa.Q),
                       dim3(SEL_THREADS), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  return hipSuccess;
}

}  // namespace csa2
