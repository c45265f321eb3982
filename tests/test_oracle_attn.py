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
