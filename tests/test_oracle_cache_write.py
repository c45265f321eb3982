"""Pins of the oracle's Full-layer cache write: RMSNorm, RoPE, the E2M1 and
E4M3 encoders, the quantizers and the entry bookkeeping of the m = 2 pair
rule (CSA2 deep-dive page, "per-layer attention computation" item 3 and "the
pool does not reduce storage"; three-modes page, Q&A on index K; V4.1-Flash
report reading, section 6)."""
import math

import numpy as np
import torch

import oracle
import synth


def _table(n_pos, base=10000.0):
    f = base ** (-np.arange(32) * 2.0 / 64.0)
    ang = np.arange(n_pos)[:, None] * f[None, :]
    return np.cos(ang), np.sin(ang)


# --------------------------------------------------------------------------
# RMSNorm and RoPE
# --------------------------------------------------------------------------

def test_rms_norm_closed_forms():
    w = np.linspace(0.5, 1.5, 8)
    # a constant row a * 1 has mean square a^2
    got = oracle.rms_norm(np.full(8, -3.0), w, 0.25)
    assert np.allclose(got, -3.0 / math.sqrt(9.25) * w, rtol=1e-15)
    # one spike s in d dims: mean square is s^2 / d (a mean, not a sum)
    x = np.zeros(8)
    x[5] = 4.0
    got = oracle.rms_norm(x, np.ones(8), 0.0)
    assert got[5] == 4.0 / math.sqrt(2.0) and np.count_nonzero(got) == 1


def test_rope_tail_by_hand():
    """Only the last 2 * len(cos) dims turn, in adjacent pairs (2j, 2j+1):
    a quarter turn maps (a, b) to (-b, a)."""
    x = np.arange(1.0, 9.0)              # dims 0..7; dims 4..7 rotate
    got = oracle.rope_tail(x, np.array([0.0, 1.0]), np.array([1.0, 0.0]))
    assert list(got) == [1, 2, 3, 4, -6, 5, 7, 8]
    got = oracle.rope_tail(x, np.array([-1.0, 0.0]), np.array([0.0, -1.0]))
    assert list(got) == [1, 2, 3, 4, -5, -6, 8, -7]


def test_rope_tail_composes_and_keeps_norm():
    rng = np.random.default_rng(2)
    x = rng.normal(size=128)
    a1, a2 = rng.uniform(-3, 3, size=32), rng.uniform(-3, 3, size=32)
    once = oracle.rope_tail(x, np.cos(a1 + a2), np.sin(a1 + a2))
    twice = oracle.rope_tail(oracle.rope_tail(x, np.cos(a1), np.sin(a1)),
                             np.cos(a2), np.sin(a2))
    assert np.allclose(once, twice, atol=1e-13)
    assert math.isclose(np.linalg.norm(once), np.linalg.norm(x), rel_tol=1e-13)
    back = oracle.rope_tail(once, np.cos(a1 + a2), -np.sin(a1 + a2))
    assert np.allclose(back, x, atol=1e-13)


# --------------------------------------------------------------------------
# Encoders (OCP MX specification: E2M1 and E4M3FN, round to nearest even,
# saturating)
# --------------------------------------------------------------------------

def test_encode_e2m1_grid_ties_and_saturation():
    grid = oracle.E2M1_TABLE[:8]
    assert list(oracle.encode_e2m1(grid)) == list(range(8))
    assert list(oracle.encode_e2m1(-grid[1:])) == list(range(9, 16))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # each midpoint goes to the neighbour with an even code
    assert list(oracle.encode_e2m1(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.encode_e2m1([6.5, 1e9, -7.0])) == [7, 7, 15]
    assert list(oracle.encode_e2m1([0.2501, 0.7499, 4.9999, 5.0001])) == [1, 1, 6, 7]


def test_encode_e2m1_agrees_with_generator_encoder():
    """The input generator's threshold encoder is written separately."""
    y = torch.randn(20000, generator=torch.Generator().manual_seed(4)) * 3
    ref = synth.formats._e2m1_codes(y.clamp(-6, 6)).numpy()
    got = oracle.encode_e2m1(y.double().numpy())
    assert np.array_equal(ref, got)


def test_encode_e4m3_round_trip_ties_and_torch():
    codes = np.arange(127, dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3(oracle.E4M3_TABLE[codes]), codes)
    assert np.array_equal(oracle.encode_e4m3(-oracle.E4M3_TABLE[codes[1:]]), codes[1:] | 0x80)
    v = oracle.E4M3_TABLE[:127]
    mids = (v[:-1] + v[1:]) / 2
    got = oracle.encode_e4m3(mids)
    lo = np.arange(126)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert list(oracle.encode_e4m3([460.0, 1e6, -500.0])) == [0x7E, 0x7E, 0xFE]
    # library cross-check: torch's round-to-nearest-even float8 conversion
    x = torch.randn(50000, generator=torch.Generator().manual_seed(6)) * 60
    x = x.clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode_e4m3(x.double().numpy())
    nz = x.numpy() != 0
    assert np.array_equal(ref[nz], got[nz])


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def test_fp4_records_agree_with_generator_and_bound_the_error():
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(7)) * 2
    ref = synth.encode_fp4_records(x).numpy()
    got = oracle.fp4_records(x.double().numpy())
    assert np.array_equal(ref, got)
    dec = oracle.decode_fp4_records(got)
    scale = np.repeat(got[:, 256:].copy().view("<f4").astype(np.float64), 32, axis=1)
    err = np.abs(dec - x.double().numpy())
    # the widest gap of the E2M1 grid is 2 (between 4 and 6)
    assert np.all(err <= scale * 1.0 + 1e-12)
    # each group's largest magnitude lands on +-6 * scale
    g = np.abs(x.double().numpy()).reshape(64, 16, 32)
    assert np.allclose(np.abs(dec).reshape(64, 16, 32).max(axis=2), g.max(axis=2), rtol=1e-6)


def test_fp4s16_records_agree_with_generator():
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(8))
    ref = synth.encode_fp4s16_records(x).numpy()
    got = oracle.fp4s16_records(x.double().numpy())
    assert np.array_equal(ref, got)


def test_fp4s16_scale_rules():
    x = np.zeros((1, 32))
    x[0, 16:] = 1e-4                  # amax / 6 is below the smallest E4M3 value
    x[0, 17] = -1.2e-4
    codes, sc = oracle.quantize_e2m1_e4m3s16(x)
    assert list(sc[0]) == [0x38, 0x01]
    assert np.all(codes[0, :16] == 0)
    # 1.2e-4 / 2^-9 = 0.06 rounds to zero, keeping the sign bit
    assert codes[0, 17] == 0x8
    y = np.full((1, 16), 3.0)
    y[0, 3] = 12.0                    # amax / 6 = 2.0 exactly: scale byte 0x40
    codes, sc = oracle.quantize_e2m1_e4m3s16(y)
    assert sc[0, 0] == 0x40 and codes[0, 3] == 7 and codes[0, 0] == 3   # 6 and 1.5


def test_fp8_rows_quantizer():
    x = np.zeros((2, 128))
    x[0, 0], x[0, 1], x[0, 2] = 896.0, -1.0, 0.3
    codes, scale = oracle.quantize_fp32_scaled(x, 128, "e4m3")
    assert scale[0] == 2.0 and scale[1] == 1.0
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0xB0   # 448 and -0.5
    assert np.all(codes[1] == 0)
    # 0.15 lies between E4M3 values 0.140625 and 0.15625: nearer the upper
    assert oracle.E4M3_TABLE[codes[0, 2]] == 0.15625


# --------------------------------------------------------------------------
# The cache write
# --------------------------------------------------------------------------

def _call(c, z, seq, pos, ratio, n_seq, pend=None, w_ik=None, kvw=None, kw=None,
          eps=1e-6, n_pos=64):
    cos, sin = _table(n_pos)
    if w_ik is None:
        w_ik = np.random.default_rng(9).normal(size=(128, 512)) / 23
    kvw = np.ones(512) if kvw is None else kvw
    kw = np.ones(128) if kw is None else kw
    pc, pz = (None, None) if pend is None else pend
    return oracle.cache_write(c, z, np.array(seq), np.array(pos), ratio, n_seq, pc, pz,
                              kvw, w_ik, kw, eps, cos, sin), (cos, sin)


def test_cache_write_ratio_one_closed_form():
    """m = 1: the entry is RMSNorm(c); with W_IK picking dims 0..127 the index
    key is RMSNorm of those dims, rotated in its last 64."""
    rng = np.random.default_rng(10)
    c = rng.normal(size=(3, 512))
    w = np.zeros((128, 512))
    w[np.arange(128), np.arange(128)] = 1.0
    kvw = rng.uniform(0.8, 1.2, size=512)
    (ent, main, k, _, _), (cos, sin) = _call(c, None, [0, 0, 1], [4, 5, 9], 1, 2,
                                             w_ik=w, kvw=kvw, eps=0.0)
    assert ent == [(0, 4), (0, 5), (1, 9)]
    for i, (t, p) in enumerate([(0, 4), (1, 5), (2, 9)]):
        u = c[t] / math.sqrt(np.mean(c[t] ** 2)) * kvw
        assert np.allclose(main[i, :448], u[:448], rtol=1e-13)
        a, b = u[448::2], u[449::2]
        assert np.allclose(main[i, 448::2], a * cos[p] - b * sin[p], atol=1e-13)
        assert np.allclose(main[i, 449::2], a * sin[p] + b * cos[p], atol=1e-13)
        kk = u[:128] / math.sqrt(np.mean(u[:128] ** 2))
        assert np.allclose(k[i, :64], kk[:64], rtol=1e-13)
        assert np.allclose(k[i, 64::2], kk[64::2] * cos[p] - kk[65::2] * sin[p], atol=1e-13)


def test_cache_write_projects_the_latent_before_rope():
    """W_IK picking dims 384..511 (the rotated ones among them) must see the
    unrotated latent."""
    rng = np.random.default_rng(11)
    c = rng.normal(size=(1, 512))
    w = np.zeros((128, 512))
    w[np.arange(128), 384 + np.arange(128)] = 1.0
    (ent, main, k, _, _), (cos, sin) = _call(c, None, [0], [7], 1, 1, w_ik=w, eps=0.0)
    u = c[0] / math.sqrt(np.mean(c[0] ** 2))
    pre = u[384:] / math.sqrt(np.mean(u[384:] ** 2))
    want = oracle.rope_tail(pre, cos[7], sin[7])
    assert np.allclose(k[0], want, atol=1e-13)
    post = main[0, 384:] / math.sqrt(np.mean(main[0, 384:] ** 2))
    assert not np.allclose(k[0], oracle.rope_tail(post, cos[7], sin[7]), atol=1e-3)


def test_cache_write_pair_softmax_is_over_tokens():
    rng = np.random.default_rng(12)
    c = rng.normal(size=(2, 512))
    z = np.zeros((2, 512))
    z[0, :256] = 60.0          # first half of the channels: token 0 dominates
    z[1, 256:] = 60.0          # second half: token 1 dominates
    (ent, main, _, _, _), _ = _call(c, z, [0, 0], [0, 1], 2, 1, eps=0.0)
    assert ent == [(0, 0)]
    mix = np.concatenate([c[0, :256], c[1, 256:]])
    u = mix / math.sqrt(np.mean(mix ** 2))
    assert np.allclose(main[0, :448], u[:448], rtol=1e-12)      # RoPE position 0
    z_eq = np.ones((2, 512)) * 0.7
    (_, main2, _, _, _), _ = _call(c, z_eq, [0, 0], [0, 1], 2, 1, eps=0.0)
    avg = (c[0] + c[1]) / 2
    assert np.allclose(main2[0, :448], (avg / math.sqrt(np.mean(avg ** 2)))[:448], rtol=1e-12)


def test_cache_write_odd_length_and_entry_positions():
    """CSA2 page: with m = 2 a sequence of N tokens holds N // 2 entries; entry
    e comes from tokens 2e, 2e+1 and (reading) turns at position 2e."""
    rng = np.random.default_rng(13)
    c, z = rng.normal(size=(7, 512)), rng.normal(size=(7, 512))
    pend = (np.zeros((1, 512)), np.zeros((1, 512)))
    (ent, main, _, pc, pz), (cos, sin) = _call(c, z, [0] * 7, list(range(7)), 2, 1, pend=pend)
    assert ent == [(0, 0), (0, 1), (0, 2)]
    assert np.array_equal(pc[0], c[6]) and np.array_equal(pz[0], z[6])
    u = oracle.rms_norm(oracle.compress(c[2:4], z[2:4], 2)[0], np.ones(512), 1e-6)
    assert np.allclose(main[1], oracle.rope_tail(u, cos[2], sin[2]), atol=1e-13)


def test_cache_write_chunked_equals_whole():
    """Splitting a sequence's tokens over calls, with the pending row carried,
    writes the same entries as one call."""
    rng = np.random.default_rng(14)
    c, z = rng.normal(size=(10, 512)), rng.normal(size=(10, 512))
    pos = list(range(10))
    (ent, main, k, _, _), _ = _call(c, z, [0] * 10, pos, 2, 1)
    pend = (np.zeros((1, 512)), np.zeros((1, 512)))
    got_e, got_m, got_k = [], [], []
    for lo, hi in [(0, 3), (3, 4), (4, 5), (5, 10)]:
        (e, m_, k_, pc, pz), _ = _call(c[lo:hi], z[lo:hi], [0] * (hi - lo), pos[lo:hi], 2, 1,
                                       pend=pend)
        pend = (pc, pz)
        got_e += e
        got_m.append(m_)
        got_k.append(k_)
    assert got_e == ent
    assert np.array_equal(np.concatenate(got_m), main)
    assert np.array_equal(np.concatenate(got_k), k)


def test_cache_write_decode_batch_and_skips():
    """One token per sequence: odd positions close a pair with the pending
    row, even positions only refresh it; bad ids and positions write nothing."""
    rng = np.random.default_rng(15)
    c, z = rng.normal(size=(5, 512)), rng.normal(size=(5, 512))
    pc, pz = rng.normal(size=(3, 512)), rng.normal(size=(3, 512))
    seq = [0, 1, 2, 3, 2]
    pos = [5, 8, 3, -1, 71]
    (ent, main, _, nc, nz), (cos, sin) = _call(c, z, seq, pos, 2, 3, pend=(pc, pz))
    # sequence 3 is out of range; sequence 2's token at 71 would close entry
    # 35, which turns at 70, outside the 64-row table
    assert ent == [(0, 2), (2, 1)]
    u = oracle.rms_norm(oracle.compress(np.stack([pc[0], c[0]]), np.stack([pz[0], z[0]]), 2)[0],
                        np.ones(512), 1e-6)
    assert np.allclose(main[0], oracle.rope_tail(u, cos[4], sin[4]), atol=1e-13)
    assert np.array_equal(nc[1], c[1]) and np.array_equal(nz[1], z[1])
    assert np.array_equal(nc[0], pc[0]) and np.array_equal(nc[2], pc[2])


# --------------------------------------------------------------------------
# Serving-shaped I/O (DSA page, top-k section; CSA2 core formula)

def test_slots_from_positions_by_hand():
    table = np.array([[3, 0, 7], [5, -1, 2]])
    idx = np.array([[0, 63, 64, 130, -1], [1, 70, 128, 191, 200]])
    got = oracle.slots_from_positions(idx, np.array([0, 1]), table)
    assert got.tolist() == [[192, 255, 0, 450, -1],
                            [321, -1, 128, 191, -1]]   # page -1 and a page past the row


def test_slots_of_an_identity_table_are_flat_rows():
    rng = np.random.default_rng(16)
    B, n_pages = 3, 5
    table = np.arange(B * n_pages).reshape(B, n_pages)
    idx = rng.integers(-1, n_pages * 64, size=(6, 40))
    q_seq = np.array([0, 1, 2, 2, 1, 0])
    got = oracle.slots_from_positions(idx, q_seq, table)
    want = np.where(idx >= 0, q_seq[:, None] * n_pages * 64 + idx, -1)
    assert np.array_equal(got, want)


def test_unturn_gives_the_relative_turn():
    """A key turned at position s, attended from position t and turned back
    there, is turned by the angle difference s - t."""
    cos, sin = _table(300)
    rng = np.random.default_rng(17)
    v = rng.normal(size=(1, 2, 512))
    s_pos, t_pos = 37, 251
    keyed = oracle.rope_tail(v, cos[s_pos], sin[s_pos])
    got = oracle.unturn_heads(keyed, np.array([t_pos]), cos, sin)
    f = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)
    d = (s_pos - t_pos) * f
    want = oracle.rope_tail(v, np.cos(d), np.sin(d))
    assert np.allclose(got, want, atol=1e-12)
    assert np.array_equal(got[0, :, :448], v[0, :, :448])
    # outside the table: unchanged
    assert np.array_equal(oracle.unturn_heads(keyed, np.array([300]), cos, sin), keyed)
