"""Pins of the oracle's sparse attention."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_closed_form_golden():
    g = json.load(open(os.path.join(GOLD, "attention_closed_form.json")))
    q = np.array(g["q"])[None]                      # [1, H=1, D=2]
    swa = np.array([g["swa_key"]])
    main = np.array([g["main_key"]])
    out, lse = oracle.sparse_attn(q, main, [0], np.array([[0]]), swa, [0], [0], None,
                                  128, [0], [0], np.array(g["sink"]), 1.0)
    assert np.allclose(out[0], g["expect_out"], rtol=1e-14)
    assert np.allclose(lse[0], g["expect_lse"], rtol=1e-14)


def _case(seed, H=4, D=16, N=40, n_swa=10, k=6):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(2, H, D))
    main = rng.normal(size=(2 * N, D))
    swa = rng.normal(size=(2 * n_swa, D))
    sink = rng.normal(size=H)
    q_seq = np.array([0, 1])
    q_pos = np.array([N - 1, N - 3])
    main_base = np.array([0, N])
    swa_pos0 = q_pos - (n_swa - 1)
    swa_base = np.array([0, n_swa])
    idx = np.full((2, k), -1)
    idx[0, :k] = np.sort(rng.choice(N, k, replace=False))
    idx[1, :k - 2] = np.sort(rng.choice(N - 2, k - 2, replace=False))
    return dict(q=q, main=main, swa=swa, sink=sink, q_seq=q_seq, q_pos=q_pos,
                main_base=main_base, swa_pos0=swa_pos0, swa_base=swa_base, idx=idx)


def _run(c, window, scale, sink=None, lo=None):
    return oracle.sparse_attn(c["q"], c["main"], c["main_base"], c["idx"], c["swa"],
                              c["swa_base"], c["swa_pos0"], lo, window, c["q_seq"],
                              c["q_pos"], c["sink"] if sink is None else sink, scale)


@pytest.mark.parametrize("window", [1, 4, 10])
def test_matches_dense_masked_softmax(window):
    """Brute force: a dense score matrix over every SWA row and every main row
    of the sequence, -inf outside the chosen set, plus one sink column whose
    value row is zero; a plain softmax over all of it."""
    c = _case(1)
    scale = 0.3
    out, lse = _run(c, window, scale)
    H, D = c["q"].shape[1:]
    for t in range(2):
        b, p = c["q_seq"][t], c["q_pos"][t]
        swa_all = c["swa"][c["swa_base"][b]:c["swa_base"][b] + 10]
        swa_pos = c["swa_pos0"][b] + np.arange(10)
        main_all = c["main"][c["main_base"][b]:c["main_base"][b] + 40]
        keys = np.concatenate([swa_all, main_all, np.zeros((1, D))])
        mask = np.concatenate([(swa_pos >= p - window + 1) & (swa_pos <= p),
                               np.isin(np.arange(40), c["idx"][t][c["idx"][t] >= 0]),
                               [True]])
        for h in range(H):
            z = scale * keys[:-1] @ c["q"][t, h]
            z = np.append(z, c["sink"][h])
            z[~mask] = -np.inf
            pr = np.exp(z - z.max())
            pr /= pr.sum()
            assert np.allclose(out[t, h], pr @ keys, rtol=1e-12, atol=1e-13)
            zf = z[mask]
            assert math.isclose(lse[t, h], zf.max() + math.log(np.exp(zf - zf.max()).sum()),
                                rel_tol=1e-13)


def test_no_sink_matches_torch_sdpa():
    """With the sink at -inf the result is ordinary attention over the chosen
    keys (library cross-check with torch's scaled_dot_product_attention)."""
    c = _case(2)
    out, _ = _run(c, 5, 0.25, sink=np.full(4, -np.inf))
    for t in range(2):
        K = oracle.attention_keys(t, c["main"], c["main_base"], c["idx"], c["swa"],
                                  c["swa_base"], c["swa_pos0"], None, 5, c["q_seq"], c["q_pos"])
        qt = torch.from_numpy(c["q"][t])[None]                    # [1, H, D]
        kt = torch.from_numpy(K)[None, None].expand(1, 4, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[:, :, None, :], kt, kt, scale=0.25)[0, :, 0, :].numpy()
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-13)


def test_sink_closed_form():
    """o_sink = o_nosink * S / (S + exp(s)), S = sum_j exp(z_j)."""
    c = _case(3)
    scale = 0.2
    o_sink, lse_sink = _run(c, 10, scale)
    o_plain, lse_plain = _run(c, 10, scale, sink=np.full(4, -np.inf))
    S = np.exp(lse_plain)
    ratio = S / (S + np.exp(c["sink"])[None, :])
    assert np.allclose(o_sink, o_plain * ratio[:, :, None], rtol=1e-12, atol=1e-14)
    assert np.allclose(np.exp(lse_sink), S + np.exp(c["sink"])[None, :], rtol=1e-12)


def test_duplicate_position_counts_twice():
    """A position in both the window and the main selection contributes its
    SWA vector and its main vector (different projections)."""
    D = 3
    q = np.array([[[1.0, 0.0, 0.0]]])
    swa = np.array([[0.0, 1.0, 0.0]])
    main = np.array([[0.0, 0.0, 1.0]])
    out, _ = oracle.sparse_attn(q, main, [0], np.array([[0]]), swa, [0], [0], None, 128,
                                [0], [0], np.array([-np.inf]), 1.0)
    assert np.allclose(out[0, 0], [0.0, 0.5, 0.5])


def test_window_lower_clamp():
    """CSA2 page, 'CED': bounded replay truncates the window at the replay
    start s, so the query at i sees [max(s, i-W+1), i]."""
    c = _case(4)
    full, _ = _run(c, 10, 0.3, lo=np.array([0, 0]))
    clamp, _ = _run(c, 10, 0.3, lo=np.array([c["q_pos"][0] - 2, 0]))
    assert not np.allclose(full[0], clamp[0]) and np.allclose(full[1], clamp[1])
    K = oracle.attention_keys(0, c["main"], c["main_base"], c["idx"], c["swa"], c["swa_base"],
                              c["swa_pos0"], np.array([c["q_pos"][0] - 2, 0]), 10,
                              c["q_seq"], c["q_pos"])
    assert K.shape[0] == 3 + 6


def test_empty_key_set_gives_zero():
    q = np.ones((1, 2, 4))
    out, lse = oracle.sparse_attn(q, np.zeros((1, 4)), [0], np.array([[-1, -1]]),
                                  np.zeros((1, 4)), [0], [0], None, 0, [0], [0],
                                  np.array([0.0, 1.0]), 1.0)
    assert np.all(out == 0) and np.allclose(lse, [0.0, 1.0])


def _dense_reference(q, keys, mask, sink, scale):
    """Plain softmax over every candidate key row with -inf outside `mask`,
    plus one sink column whose value row is zero: [H, D]."""
    H, D = q.shape
    allk = np.concatenate([keys, np.zeros((1, D))])
    m = np.append(mask, True)
    out = np.zeros((H, D))
    for h in range(H):
        z = np.append(scale * keys @ q[h], sink[h])
        z[~m] = -np.inf
        pr = np.exp(z - z.max())
        out[h] = (pr / pr.sum()) @ allk
    return out


@pytest.mark.parametrize("ratio", [1, 2])
def test_invalid_indices_name_no_key(ratio):
    """Reading 22: an idx entry that is negative or at/after the query's
    visible count (p+1)//m names no key.  Brute force: a dense mask over every
    main row of the sequence, built from the entries that lie in [0, n_vis),
    gives the same output; and replacing the invalid entries by -1 changes
    nothing.  The entries n_vis - 1 (kept) and n_vis (dropped) pin the
    boundary."""
    rng = np.random.default_rng(11)
    H, D, N = 3, 8, 50
    p = 37
    n_vis = (p + 1) // ratio
    q = rng.normal(size=(1, H, D))
    main = rng.normal(size=(N, D))
    swa = rng.normal(size=(4, D))
    sink = rng.normal(size=H)
    idx = np.array([[2, n_vis - 1, n_vis, n_vis + 5, N - 1, -1, -7, 5]])
    args = dict(main_rows=main, main_base=[0], swa_rows=swa, swa_base=[0], swa_pos0=[p - 3],
                swa_lo=None, window=4, q_seq=[0], q_pos=[p], sink=sink, scale=0.4, ratio=ratio)
    out, _ = oracle.sparse_attn(q, idx=idx, **args)
    clean = np.where((idx >= 0) & (idx < n_vis), idx, -1)
    out_clean, _ = oracle.sparse_attn(q, idx=clean, **args)
    assert np.array_equal(out, out_clean)
    keys = np.concatenate([swa, main])
    mask = np.concatenate([np.ones(4, bool),
                           np.isin(np.arange(N), [2, n_vis - 1, 5]) & (np.arange(N) < n_vis)])
    assert np.allclose(out[0], _dense_reference(q[0], keys, mask, sink, 0.4), rtol=1e-12, atol=1e-13)
    K = oracle.attention_keys(0, main, [0], idx, swa, [0], [p - 3], None, 4, [0], [p], ratio)
    assert K.shape[0] == 4 + 3


@pytest.mark.parametrize("pos0_offset,lo_offset,expect_swa", [
    (0, None, 10),      # every stored row inside the window
    (4, None, 6),       # oldest stored row after p - W + 1: the window starts there
    (4, 7, 3),          # replay start after the stored rows: it wins
    (4, 10, 0),         # replay start past p: no SWA key at all
    (0, 2, 8),          # replay start inside the window
])
def test_window_starts_at_latest_of_replay_stored_and_window(pos0_offset, lo_offset, expect_swa):
    """CSA2 page, 'CED' (bounded replay): the query at p sees the SWA keys of
    [max(s, p-W+1), p].  Rows before the oldest stored position swa_pos0 do
    not exist and are skipped (the stored rows start at swa_base).  Brute
    force over the stored rows with an explicit position mask."""
    rng = np.random.default_rng(12)
    H, D, W = 2, 6, 10
    p = 40
    pos0 = p - W + 1 + pos0_offset
    n_stored = p - pos0 + 1
    q = rng.normal(size=(1, H, D))
    swa = rng.normal(size=(3 + n_stored, D))      # three rows of another sequence first
    main = rng.normal(size=(20, D))
    sink = rng.normal(size=H)
    idx = np.array([[3, 9, -1]])
    lo = None if lo_offset is None else np.array([p - W + 1 + lo_offset])
    out, _ = oracle.sparse_attn(q, main, [0], idx, swa, [3], [pos0], lo, W, [0], [p], sink, 0.5)
    K = oracle.attention_keys(0, main, [0], idx, swa, [3], [pos0], lo, W, [0], [p])
    assert K.shape[0] == expect_swa + 2
    pos = pos0 + np.arange(n_stored)
    start = p - W + 1 if lo is None else max(p - W + 1, int(lo[0]))
    keys = np.concatenate([swa[3:], main])
    mask = np.concatenate([(pos >= start) & (pos <= p), np.isin(np.arange(20), [3, 9])])
    assert mask[:n_stored].sum() == expect_swa
    assert np.allclose(out[0], _dense_reference(q[0], keys, mask, sink, 0.5), rtol=1e-12, atol=1e-13)
