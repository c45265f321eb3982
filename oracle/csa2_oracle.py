"""CPU oracle for the CSA2 global-attention hot path (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The library (the HIP path) never
calls it and shares no code with it: this file has its own format decoders,
its own selection routines and its own attention.

Sources, cited as page + section (the pages are Chinese-language web pages):

  [CSA2]    zdszero.github.io/csa2.html, the CSA2 deep-dive
  [3MODES]  xhh.club, "DeepSeek-V4.1 model structure (2): CSA2's three modes"
  [REPORT]  10100.com, "DeepSeek-V4.1-Flash technical report reading"
  [DSA]     zdszero.github.io/dsa.html, DeepSeek Sparse Attention (V3.2)
  [OCP-MX]  OCP Microscaling formats (arXiv:2310.10537), cited by [REPORT]'s
            references for the FP4 format; it also defines E4M3 and E2M1.

Every step reaches its plain definition exactly (up to float64 rounding); the
readings taken where the pages are silent are listed next to each function.
All inputs are NumPy arrays; nothing here touches a GPU.
"""
import math

import numpy as np

NEG_INF = -np.inf

# ----------------------------------------------------------------------------
# Format decoders ([OCP-MX]; [DSA] "two KV caches"; [CSA2] "where attention is
# computed"; [REPORT] section 6)
# ----------------------------------------------------------------------------


def e4m3_value(code):
    """OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
    field 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; no infinities.
    Largest finite magnitude 448 (the value [REPORT] section 6 multiplies by 6
    to get the 2688 headroom figure)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, -6)
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


def e2m1_value(code):
    """OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent
    field 0 is subnormal (0.5 * m).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = math.ldexp(1.0 + m / 2.0, e - 1)
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_bf16(bits):
    """bf16 bit patterns (int16/uint16) -> float64: the pattern is the upper
    half of an IEEE binary32."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def decode_e4m3_rows(codes, scale):
    """E4M3 codes [..., d] times one fp32 scale per row [...] -> float64."""
    v = E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    return v * np.asarray(scale, dtype=np.float64)[..., None]


def decode_fp4_records(rec):
    """320-byte main-KV records [n, 320] -> float64 [n, 512].
    Bytes 0..255 hold E2M1 pairs, element 2i in the low nibble of byte i;
    bytes 256..319 hold 16 little-endian fp32 scales, one per 32 elements."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    lo = rec[:, :256] & 0xF
    hi = rec[:, :256] >> 4
    codes = np.empty((n, 512), dtype=np.uint8)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    scale = rec[:, 256:320].copy().view("<f4").astype(np.float64)   # [n, 16]
    return E2M1_TABLE[codes] * np.repeat(scale, 32, axis=1)


def decode_fp4s16_rows(codes, scales):
    """FP4 rows in the pages' cache format ([REPORT] section 6: E2M1 elements
    with one E4M3 scale per 16 channels and no second-level scale):
    codes [n, d/2] (element 2i in the low nibble of byte i) and E4M3 scale
    bytes [n, d/16] -> float64 [n, d]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n, half = codes.shape
    e = np.empty((n, 2 * half), dtype=np.uint8)
    e[:, 0::2] = codes & 0xF
    e[:, 1::2] = codes >> 4
    return E2M1_TABLE[e] * np.repeat(E4M3_TABLE[scales], 16, axis=1)


def decode_fp4s16_records(rec):
    """The pages' 288-byte main-KV records [n, 288] -> float64 [n, 512]:
    256 bytes of E2M1 pairs, then 32 E4M3 scale bytes, one per 16 elements
    ([CSA2] SGLang section: 256 B of data + 32 B of scale)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    return decode_fp4s16_rows(rec[:, :256], rec[:, 256:288])


def decode_swa_records(rec):
    """528-byte SWA records [n, 528] -> float64 [n, 512]: 512 E4M3 codes, then
    4 little-endian fp32 scales, one per 128 elements."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    scale = rec[:, 512:528].copy().view("<f4").astype(np.float64)   # [n, 4]
    return E4M3_TABLE[rec[:, :512]] * np.repeat(scale, 128, axis=1)


# ----------------------------------------------------------------------------
# Visibility ([CSA2] "the pool does not reduce storage": with ratio m a main
# entry exists once m tokens are complete, so the visible count is (pos+1)//m)
# ----------------------------------------------------------------------------


def visible_count(q_pos, ratio):
    return (np.asarray(q_pos, dtype=np.int64) + 1) // int(ratio)


# ----------------------------------------------------------------------------
# Lightning-Indexer scores ([CSA2] "per-layer attention computation", item 4:
# I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]), 32 heads x 128 dims;
# [DSA] "Lightning Indexer" for the same formula)
#
# Reading: no 1/sqrt(d) or 1/sqrt(H) factor appears in the formula; any such
# factor belongs to the caller and is folded into w ([DSA] "fp8 and scale
# absorption" folds them into the gates).  q and k are the dequantized values.
# ----------------------------------------------------------------------------


def index_scores_dense(q, w, k_rows, seq_base, q_seq, q_pos, ratio, n_cols):
    """q [Q, H, d], w [Q, H], k_rows [sum N, d] (all float64).
    Returns [Q, n_cols]: the score for s < min(visible, n_cols), -inf after."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Q = q.shape[0]
    out = np.full((Q, n_cols), NEG_INF)
    nvis = visible_count(q_pos, ratio)
    for t in range(Q):
        n = int(min(nvis[t], n_cols))
        if n <= 0:
            continue
        base = int(seq_base[int(q_seq[t])])
        keys = np.asarray(k_rows[base:base + n], dtype=np.float64)   # [n, d]
        dots = q[t] @ keys.T                                         # [H, n]
        out[t, :n] = w[t] @ np.maximum(dots, 0.0)
    return out


def pool_positions(cand, block_size):
    """Compact pool order: entry c*bs + j is position cand[c]*bs + j, or -1
    where cand[c] is -1 ([CSA2] "hierarchical sparse indexer": the pool is
    the positions covered by the chosen blocks)."""
    cand = np.asarray(cand, dtype=np.int64)
    pos = cand[..., :, None] * block_size + np.arange(block_size)
    pos = np.where(cand[..., :, None] >= 0, pos, -1)
    return pos.reshape(cand.shape[:-1] + (cand.shape[-1] * block_size,))


def index_scores_pool(q, w, k_rows, seq_base, q_seq, q_pos, ratio, cand, block_size):
    """Scores only at the pool positions, in compact candidate order
    ([CSA2] "where attention is computed": the candidate indexer computes
    logits only for the candidate blocks; [REPORT] section 5).  Entries whose
    block is -1 or whose position is not visible are -inf."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Q = q.shape[0]
    pos = pool_positions(cand, block_size)                 # [Q, nb*bs]
    out = np.full(pos.shape, NEG_INF)
    nvis = visible_count(q_pos, ratio)
    for t in range(Q):
        ok = (pos[t] >= 0) & (pos[t] < nvis[t])
        if not ok.any():
            continue
        base = int(seq_base[int(q_seq[t])])
        keys = np.asarray(k_rows[base + pos[t][ok]], dtype=np.float64)
        out[t, ok] = w[t] @ np.maximum(q[t] @ keys.T, 0.0)
    return out


# ----------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------


def _first_k_by_score(values, positions, k):
    """Indices (into values) of the first k entries under (value desc,
    position asc), among entries whose value is greater than -inf."""
    values = np.asarray(values, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    ok = np.nonzero(values > NEG_INF)[0]
    order = np.lexsort((positions[ok], -values[ok]))   # last key is primary
    return ok[order[:k]]


def topk(values, positions, k):
    """Token-level top-k ([CSA2] "per-layer attention computation", item 4:
    top-512 of the index scores; [DSA] "Top-k: tokens, not blocks": a
    (rows, k) int32 table padded with -1).

    Readings: ties go to the lower position; -inf entries are never chosen,
    so a row with fewer than k finite entries selects all of them ([DSA]
    "design": when S <= k top-k selects every token); the chosen positions
    are returned in ascending order, then -1 padding."""
    sel = _first_k_by_score(values, positions, k)
    chosen = np.sort(np.asarray(positions, dtype=np.int64)[sel])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


def topk_rows_dense(scores, q_pos, ratio, k):
    """Top-k of each dense score row over its visible prefix."""
    scores = np.asarray(scores, dtype=np.float64)
    Q, n_cols = scores.shape
    nvis = visible_count(q_pos, ratio)
    out = np.full((Q, k), -1, dtype=np.int64)
    for t in range(Q):
        n = int(min(nvis[t], n_cols))
        out[t] = topk(scores[t, :n], np.arange(n), k)
    return out


def topk_rows_pool(scores, cand, block_size, k):
    """Top-k of each compact pool row; positions come from the pool."""
    pos = pool_positions(cand, block_size)
    scores = np.asarray(scores, dtype=np.float64)
    out = np.full((scores.shape[0], k), -1, dtype=np.int64)
    for t in range(scores.shape[0]):
        v = np.where(pos[t] >= 0, scores[t], NEG_INF)
        out[t] = topk(v, np.maximum(pos[t], 0), k)
    return out


def block_maxima(row, n, block_size):
    """Per-block maximum of the first n entries of a score row ([CSA2]
    "blocks are not compression": a block's score is the largest index score
    inside it, not the mean).  The last block may be partial."""
    nb = -(-n // block_size)
    bm = np.full(nb, NEG_INF)
    for b in range(nb):
        bm[b] = np.max(row[b * block_size:min(n, (b + 1) * block_size)])
    return bm


def block_candidates(scores, q_pos, ratio, block_size, n_blocks):
    """Candidate pool of each query ([CSA2] "hierarchical sparse indexer",
    "which positions are in the pool", "where attention is computed";
    [REPORT] section 5): blocks of block_size positions scored by their
    maximum, the n_blocks best kept, the block holding the latest visible
    position always kept.

    Readings: the latest block is forced by giving it the score +inf before
    selection, so the pool never exceeds n_blocks blocks; ties go to the
    lower block id; blocks whose maximum is -inf are not chosen; the chosen
    block ids are returned ascending, then -1 padding."""
    scores = np.asarray(scores, dtype=np.float64)
    Q, n_cols = scores.shape
    nvis = visible_count(q_pos, ratio)
    out = np.full((Q, n_blocks), -1, dtype=np.int64)
    for t in range(Q):
        n = int(min(nvis[t], n_cols))
        if n <= 0:
            continue
        bm = block_maxima(scores[t], n, block_size)
        bm[-1] = np.inf
        out[t] = topk(bm, np.arange(len(bm)), n_blocks)
    return out


# ----------------------------------------------------------------------------
# Core sparse attention ([CSA2] "per-layer attention computation": one joint
# softmax per head over the layer's last-128 SWA keys and the selected main
# keys, divided by sqrt(d), with a per-head sink that enters only the
# denominator; MQA with K = V; [3MODES] Q&A on Reuse layers)
#
# Readings: scale = 1/sqrt(512) by default (the head dim); the sink is a raw
# logit s_i (not scaled); the SWA window of the query at token position p is
# [max(lo, p-W+1), p] including p itself ([CSA2] "CED" bounded replay gives
# the lo clamp, lo = 0 when absent); a position present both in the window and
# among the main keys contributes twice, since the two are different vectors
# ([CSA2] "per-layer attention computation": with m = 1 a token has an SWA KV
# and a main KV from different projections).
# ----------------------------------------------------------------------------


def attention_keys(t, main_rows, main_base, idx, swa_rows, swa_base, swa_pos0,
                   swa_lo, window, q_seq, q_pos, ratio=1):
    """Key matrix of query t: SWA rows (oldest first), then main rows.
    Readings: an idx entry that is negative or not visible to the query
    ((pos+1)//ratio or beyond) names no key; SWA positions below swa_pos0[b]
    (rows the caller does not hold) are not in the window."""
    b = int(q_seq[t])
    p = int(q_pos[t])
    lo = 0 if swa_lo is None else int(swa_lo[b])
    # the window starts at the replay start, at the oldest stored SWA row
    # (position swa_pos0[b]) and at position 0, whichever is latest
    first = max(lo, int(swa_pos0[b]), p - window + 1, 0)
    swa_idx = int(swa_base[b]) + np.arange(first, p + 1) - int(swa_pos0[b])
    sel = np.asarray(idx[t], dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < (p + 1) // int(ratio))]
    main_idx = int(main_base[b]) + sel
    return np.concatenate([np.asarray(swa_rows[swa_idx], dtype=np.float64),
                           np.asarray(main_rows[main_idx], dtype=np.float64)], 0)


def sparse_attn(q, main_rows, main_base, idx, swa_rows, swa_base, swa_pos0,
                swa_lo, window, q_seq, q_pos, sink, scale, ratio=1):
    """q [Q, H, D]; main_rows [sum N, D]; swa_rows [rows, D]; idx [Q, k] with
    -1 = no key; sink [H].  Returns (out [Q, H, D], lse [Q, H]) where
    lse = log(sum_j exp(z_j) + exp(sink))."""
    q = np.asarray(q, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    Q, H, D = q.shape
    out = np.zeros((Q, H, D))
    lse = np.zeros((Q, H))
    for t in range(Q):
        K = attention_keys(t, main_rows, main_base, idx, swa_rows, swa_base,
                           swa_pos0, swa_lo, window, q_seq, q_pos, ratio)   # [n, D]
        z = scale * (q[t] @ K.T)                                      # [H, n]
        zmax = z.max(axis=1) if z.shape[1] else np.full(H, NEG_INF)
        M = np.maximum(zmax, sink)
        e = np.exp(z - M[:, None])
        den = e.sum(axis=1) + np.exp(sink - M)
        out[t] = (e @ K) / den[:, None]
        lse[t] = M + np.log(den)
    return out, lse


# ----------------------------------------------------------------------------
# Compressor ([3MODES] "compression operator simplified": non-overlapping
# groups of m tokens, per-channel softmax over the group, no positional bias;
# with m = 1 the weight is identically 1 and no Z projection exists)
# ----------------------------------------------------------------------------


def compress(c, z, m):
    """c, z [T, D] -> [T // m, D]: entry i, channel ch = sum over the m tokens
    of the group of softmax_group(z)[token, ch] * c[token, ch]."""
    c = np.asarray(c, dtype=np.float64)
    T, D = c.shape
    n = T // m
    if m == 1:
        return c[:n].copy()
    z = np.asarray(z, dtype=np.float64)
    cg = c[: n * m].reshape(n, m, D)
    zg = z[: n * m].reshape(n, m, D)
    zg = zg - zg.max(axis=1, keepdims=True)
    e = np.exp(zg)
    return (e / e.sum(axis=1, keepdims=True) * cg).sum(axis=1)


# ----------------------------------------------------------------------------
# Full-layer cache write ([CSA2] "per-layer attention computation", item 3:
# the compressed entry passes RMSNorm to a latent taken before RoPE; one copy
# gets RoPE and FP4 quantization for the main-KV cache, the other is
# projected, normalised, rotated and quantized into the index key.  [3MODES]
# Q&A "how is indexer K generated": k = RMSNorm(C W_IK) with W_IK 512 x 128,
# applied to the latent before RoPE, with RoPE on the last 64 dims after the
# projection.  [REPORT] section 6: quantization comes after RoPE.  [CSA2]
# "the pool does not reduce storage": with m = 2 an entry is written only once
# both tokens of its pair exist, so n tokens hold n // 2 entries.)
#
# Readings where the pages are silent:
#  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * weight.
#  * RoPE turns adjacent pairs (2j, 2j+1) of the rotated dims by the angle of
#    frequency j, with cos/sin read from a per-position table:
#      x'[2j] = x[2j] cos_j - x[2j+1] sin_j,  x'[2j+1] = x[2j] sin_j + x[2j+1] cos_j.
#    The main latent and the index key use the same table.
#  * The RoPE position of entry e is the position of its first token, e * m.
#  * The index-key weight is stored as a linear layer's [128, 512] matrix:
#    k[n] = sum_c u[c] W[n, c].
#  * Quantization: per group, scale = amax / fmax (fmax = 6 for E2M1, 448 for
#    E4M3), kept in fp32 (1.0 for an all-zero group), or rounded to E4M3 for
#    the per-16 format (0x38 = 1.0 for an all-zero group, the smallest
#    positive E4M3 value when the rounding gives zero).  Each element becomes
#    the representable value nearest to x / scale, ties to the even code,
#    saturating at the largest magnitude.
# ----------------------------------------------------------------------------

E2M1_GRID = E2M1_TABLE[:8]     # codes 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6
E4M3_GRID = E4M3_TABLE[:127]   # codes 0..126: 0 .. 448 (0x7f is NaN)


def rms_norm(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(weight, dtype=np.float64)


def rope_tail(x, cos, sin):
    """Rotate the last 2 * len(cos) dims of x (one row, or rows with one
    cos/sin row each) in adjacent pairs."""
    x = np.array(x, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    r = 2 * cos.shape[-1]
    d = x.shape[-1]
    a = x[..., d - r::2].copy()
    b = x[..., d - r + 1::2].copy()
    x[..., d - r::2] = a * cos - b * sin
    x[..., d - r + 1::2] = a * sin + b * cos
    return x


def _nearest_index(mag, grid):
    """Index of the grid value nearest to each magnitude; at a midpoint the
    even index wins (neighbouring codes alternate their lowest bit, so this is
    ties-to-even); magnitudes beyond the top saturate to it."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    mid = (grid[lo] + grid[hi]) / 2.0
    up = (mag > mid) | ((mag == mid) & (hi % 2 == 0))
    return np.where(up, hi, lo)


def encode_e2m1(x):
    """float64 -> E2M1 codes (sign in bit 3; a negative value that rounds to
    zero keeps its sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_index(np.abs(x), E2M1_GRID).astype(np.uint8)
    return code | ((x < 0).astype(np.uint8) << 3)


def encode_e4m3(x):
    """float64 -> E4M3FN codes (sign in bit 7), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_index(np.abs(x), E4M3_GRID).astype(np.uint8)
    return code | ((x < 0).astype(np.uint8) << 7)


def quantize_fp32_scaled(x, group, kind):
    """x [n, d] -> (codes [n, d] uint8, fp32 scales [n, d // group]);
    kind 'e2m1' (fmax 6) or 'e4m3' (fmax 448)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    fmax, enc = (6.0, encode_e2m1) if kind == "e2m1" else (448.0, encode_e4m3)
    g = x.reshape(n, d // group, group)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / fmax, 1.0).astype(np.float32)
    codes = enc(g / scale.astype(np.float64)[..., None])
    return codes.reshape(n, d), scale


def quantize_e2m1_e4m3s16(x):
    """The pages' FP4 format: x [n, d] -> (E2M1 codes [n, d], E4M3 scale
    bytes [n, d // 16])."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    g = x.reshape(n, d // 16, 16)
    amax = np.abs(g).max(axis=2)
    sc = encode_e4m3(amax / 6.0)
    sc = np.where(amax == 0, 0x38, np.where(sc == 0, 0x01, sc)).astype(np.uint8)
    codes = encode_e2m1(g / E4M3_TABLE[sc][..., None])
    return codes.reshape(n, d), sc


def pack_e2m1(codes):
    """E2M1 codes [n, d] -> bytes [n, d / 2], element 2i in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def fp4_records(x):
    """[n, 512] -> 320-byte records: packed E2M1, then 16 fp32 scales."""
    codes, scale = quantize_fp32_scaled(x, 32, "e2m1")
    return np.concatenate([pack_e2m1(codes),
                           scale.astype("<f4").view(np.uint8).reshape(len(x), 64)], axis=1)


def fp4s16_records(x):
    """[n, 512] -> the pages' 288-byte records: packed E2M1, then 32 E4M3 scales."""
    codes, sc = quantize_e2m1_e4m3s16(x)
    return np.concatenate([pack_e2m1(codes), sc], axis=1)


def cache_write(c, z, tok_seq, tok_pos, ratio, n_seq, pend_c, pend_z, kv_norm_w,
                w_ik, k_norm_w, eps, rope_cos, rope_sin):
    """A Full layer's cache write for one call's tokens.

    c, z [T, 512] token rows (z is unused with ratio 1); tok_seq, tok_pos [T];
    pend_c, pend_z: None, or [n_seq, 512] rows of the token that opened each
    sequence's incomplete pair in an earlier call; w_ik [128, 512];
    rope_cos, rope_sin [n_pos, 32].

    A token at position p closes entry e = p // m when (p + 1) % m == 0.  With
    m = 2 its partner at p - 1 is the previous token of the call when that is
    the same sequence at p - 1, else the pending row; without either, or with
    the RoPE position outside the table, or with a sequence id outside
    [0, n_seq), the token writes nothing.  Returns (entries, main, k, pend_c',
    pend_z'): entries lists (seq, e) in token order, main [n, 512] and k
    [n, 128] are the post-RoPE values before quantization, and the pending
    rows are updated from the token that ends each sequence's run at an even
    position (after every entry has read the old ones)."""
    m = int(ratio)
    c = np.asarray(c, dtype=np.float64)
    z = None if z is None else np.asarray(z, dtype=np.float64)
    T = len(tok_seq)
    entries, mains, ks = [], [], []
    for t in range(T):
        s, p = int(tok_seq[t]), int(tok_pos[t])
        if s < 0 or s >= n_seq or p < 0 or (p + 1) % m:
            continue
        if m == 1:
            cg, zg = c[t:t + 1], None
        elif t > 0 and int(tok_seq[t - 1]) == s and int(tok_pos[t - 1]) == p - 1:
            cg, zg = c[t - 1:t + 1], z[t - 1:t + 1]
        elif pend_c is not None:
            cg = np.stack([np.asarray(pend_c[s], np.float64), c[t]])
            zg = np.stack([np.asarray(pend_z[s], np.float64), z[t]])
        else:
            continue
        e = p // m
        if e * m >= len(rope_cos):
            continue
        u = rms_norm(compress(cg, zg, m)[0], kv_norm_w, eps)
        main = rope_tail(u, rope_cos[e * m], rope_sin[e * m])
        k = rms_norm(u @ np.asarray(w_ik, np.float64).T, k_norm_w, eps)
        k = rope_tail(k, rope_cos[e * m], rope_sin[e * m])
        entries.append((s, e))
        mains.append(main)
        ks.append(k)
    new_c = None if pend_c is None else np.array(pend_c, dtype=np.float64)
    new_z = None if pend_z is None else np.array(pend_z, dtype=np.float64)
    if m == 2 and new_c is not None:
        for t in range(T):
            s, p = int(tok_seq[t]), int(tok_pos[t])
            if s < 0 or s >= n_seq or p < 0 or p % 2:
                continue
            last = (t == T - 1 or int(tok_seq[t + 1]) != s
                    or int(tok_pos[t + 1]) != p + 1)
            if last:
                new_c[s] = c[t]
                new_z[s] = z[t]
    main = np.array(mains).reshape(-1, c.shape[1])
    k = np.array(ks).reshape(-1, 128)
    return entries, main, k, new_c, new_z


# ----------------------------------------------------------------------------
# Layer roles and the shared slot set ([3MODES] "shared pool mechanism": the
# SharedAttentionRuntime holds four slots compress_kv, index_k, topk_idxs and
# candidates; Full writes them, Reindex rewrites topk_idxs from the pool,
# Reuse only reads; [CSA2] "three modes"; [REPORT] section 4)
# ----------------------------------------------------------------------------


def global_entries_per_token(full_layer_ratios):
    """Resident global-KV entries per token: each Full layer stores one entry
    per m tokens ([CSA2] "the pool does not reduce storage" and the V4.1-Flash
    configuration: 3 encoder Full layers at m = 2 and 1 decoder Full layer at
    m = 1)."""
    return sum(1.0 / m for m in full_layer_ratios)


def run_layers(layers, k_rows, main_rows, seq_base, q_seq, q_pos, ratio,
               swa_base, swa_pos0, window, topk_k, block_size, n_blocks, scale,
               use_pool=True):
    """Run a sequence of layers through the slot set.

    layers: list of dicts with keys mode ('full' | 'reindex' | 'reuse'),
    q [Q,H,D], swa_rows [rows,D], sink [H], and for indexer layers q_idx
    [Q,32,128] (dequantized) and w [Q,32].  Returns per-layer dicts with the
    scores, candidates, idx and attention output computed for that layer.

    Reading ([CSA2] "hierarchical sparse indexer" and "where attention is
    computed"): only a Full layer followed by a Reindex layer builds a pool;
    a Reindex layer with no pool scores every visible position."""
    slots = {"topk_idxs": None, "candidates": None}
    results = []
    n_cols = int(visible_count(q_pos, ratio).max())
    needs_pool = [any(m["mode"] == "reindex" for m in layers[i + 1:])
                  for i in range(len(layers))]
    for li, lay in enumerate(layers):
        r = {"mode": lay["mode"]}
        if lay["mode"] == "full":
            sc = index_scores_dense(lay["q_idx"], lay["w"], k_rows, seq_base,
                                    q_seq, q_pos, ratio, n_cols)
            r["scores"] = sc
            slots["topk_idxs"] = topk_rows_dense(sc, q_pos, ratio, topk_k)
            if use_pool and needs_pool[li]:
                slots["candidates"] = block_candidates(sc, q_pos, ratio,
                                                       block_size, n_blocks)
                r["candidates"] = slots["candidates"]
        elif lay["mode"] == "reindex":
            if slots["candidates"] is not None:
                sc = index_scores_pool(lay["q_idx"], lay["w"], k_rows, seq_base,
                                       q_seq, q_pos, ratio, slots["candidates"],
                                       block_size)
                slots["topk_idxs"] = topk_rows_pool(sc, slots["candidates"],
                                                    block_size, topk_k)
            else:
                sc = index_scores_dense(lay["q_idx"], lay["w"], k_rows, seq_base,
                                        q_seq, q_pos, ratio, n_cols)
                slots["topk_idxs"] = topk_rows_dense(sc, q_pos, ratio, topk_k)
            r["scores"] = sc
        r["idx"] = slots["topk_idxs"]
        r["out"], r["lse"] = sparse_attn(lay["q"], main_rows, seq_base,
                                         slots["topk_idxs"], lay["swa_rows"],
                                         swa_base, swa_pos0, None, window,
                                         q_seq, q_pos, lay["sink"], scale, ratio)
        results.append(r)
    return results


# ----------------------------------------------------------------------------
# Serving-shaped I/O ([DSA] top-k section: the KV cache is paged, so each
# selected position p becomes the physical slot table[p // 64] * 64 + p % 64
# of a 64-slot page, -1 staying -1, and the sparse kernel gathers by slot;
# [CSA2] core formula: the attention output is turned back by RoPE before
# the output projection)
#
# Readings: a page-table entry that is negative, or a page past the row's
# width, names no slot (-1).  The output's turned dims (the last 64 of each
# head) are turned back by the query's own position with the table the cache
# write used; a position outside the table leaves the output as it is.
# ----------------------------------------------------------------------------

PAGE_SLOTS = 64


def slots_from_positions(idx, q_seq, page_table):
    """idx [Q, k] positions (-1 padded), q_seq [Q], page_table [B, n_pages]
    -> [Q, k] physical slots."""
    idx = np.asarray(idx, dtype=np.int64)
    table = np.asarray(page_table, dtype=np.int64)
    out = np.full(idx.shape, -1, dtype=np.int64)
    for t in range(idx.shape[0]):
        row = table[int(q_seq[t])]
        for j in range(idx.shape[1]):
            p = int(idx[t, j])
            if p < 0 or p // PAGE_SLOTS >= len(row):
                continue
            page = int(row[p // PAGE_SLOTS])
            if page >= 0:
                out[t, j] = page * PAGE_SLOTS + p % PAGE_SLOTS
    return out


def unturn_heads(out, q_pos, rope_cos, rope_sin):
    """out [Q, H, D]: the last 64 dims of every head turned back by the
    query's position (the inverse of rope_tail at that position)."""
    out = np.array(out, dtype=np.float64)
    for t in range(out.shape[0]):
        p = int(q_pos[t])
        if 0 <= p < len(rope_cos):
            out[t] = rope_tail(out[t], rope_cos[p], -np.asarray(rope_sin[p], dtype=np.float64))
    return out
