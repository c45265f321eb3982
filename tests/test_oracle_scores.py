"""Pins of the oracle's Lightning-Indexer scores (dense and pool)."""
import numpy as np
import pytest

import oracle


def _brute_scores(q, w, k, seq_base, q_seq, q_pos, ratio, n_cols):
    """Explicit loops over query, key, head and dim."""
    Q, H, d = q.shape
    out = [[float("-inf")] * n_cols for _ in range(Q)]
    for t in range(Q):
        n = (int(q_pos[t]) + 1) // ratio
        for s in range(min(n, n_cols)):
            row = int(seq_base[int(q_seq[t])]) + s
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for j in range(d):
                    dot += q[t, h, j] * k[row, j]
                tot += w[t, h] * (dot if dot > 0 else 0.0)
            out[t][s] = tot
    return np.array(out)


@pytest.mark.parametrize("ratio", [1, 2])
def test_dense_scores_brute_force(ratio):
    rng = np.random.default_rng(11)
    H, d = 4, 5
    n_entries = [9, 6]
    seq_base = np.array([0, 9])
    q_seq = np.array([0, 0, 1])
    q_pos = np.array([17, 4, 11]) if ratio == 2 else np.array([8, 3, 5])
    q = rng.normal(size=(3, H, d))
    w = rng.normal(size=(3, H))
    k = rng.normal(size=(sum(n_entries), d))
    n_cols = 9
    ref = _brute_scores(q, w, k, seq_base, q_seq, q_pos, ratio, n_cols)
    got = oracle.index_scores_dense(q, w, k, seq_base, q_seq, q_pos, ratio, n_cols)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.allclose(got[fin], ref[fin], rtol=1e-13, atol=1e-13)


def test_dense_scores_integer_exact():
    """Integer q, k in [-4, 4] and w in [-2, 2]: the exact integer result."""
    rng = np.random.default_rng(3)
    q = rng.integers(-4, 5, size=(4, 32, 128))
    w = rng.integers(-2, 3, size=(4, 32))
    k = rng.integers(-4, 5, size=(300, 128))
    q_pos = np.array([299, 298, 150, 0])
    got = oracle.index_scores_dense(q.astype(float), w.astype(float), k.astype(float),
                                    [0], [0] * 4, q_pos, 1, 300)
    dots = np.einsum("thd,sd->ths", q, k)                      # int64
    exact = np.einsum("th,ths->ts", w, np.maximum(dots, 0))
    for t in range(4):
        n = q_pos[t] + 1
        assert np.array_equal(got[t, :n], exact[t, :n].astype(float))
        assert np.all(got[t, n:] == -np.inf)


def test_scale_folding_identity():
    """DSA page, 'fp8 and scale absorption': with positive scales,
    kscale[s] * sum_h (w*qscale)[h] * ReLU(q8 . k8) equals the score of the
    dequantized vectors, because ReLU(a x) = a ReLU(x) for a > 0."""
    rng = np.random.default_rng(5)
    q8 = rng.integers(0, 256, size=(2, 32, 128)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x10       # avoid the NaN codes
    k8 = rng.integers(0, 256, size=(50, 128)).astype(np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x21
    qs = rng.uniform(0.01, 2.0, size=(2, 32))
    ks = rng.uniform(0.01, 2.0, size=50)
    w = rng.normal(size=(2, 32))
    qv = oracle.E4M3_TABLE[q8]
    kv = oracle.E4M3_TABLE[k8]
    folded = ks[None, :] * np.einsum("th,ths->ts", w * qs,
                                     np.maximum(np.einsum("thd,sd->ths", qv, kv), 0))
    got = oracle.index_scores_dense(oracle.decode_e4m3_rows(q8, qs), w,
                                    oracle.decode_e4m3_rows(k8, ks), [0], [0, 0],
                                    [49, 49], 1, 50)
    assert np.allclose(got, folded, rtol=1e-12, atol=1e-9)


def test_visibility_rule():
    """CSA2 page, 'the pool does not reduce storage': with m = 2 an entry is
    written only when the token count is even, so an odd-length prefix leaves
    its last token without a main entry; the visible count is (pos+1)//m."""
    assert list(oracle.visible_count([0, 1, 4, 5, 6], 2)) == [0, 1, 2, 3, 3]
    assert list(oracle.visible_count([0, 7, 2047], 1)) == [1, 8, 2048]
    got = oracle.index_scores_dense(np.ones((1, 1, 1)), np.ones((1, 1)), np.ones((10, 1)),
                                    [0], [0], [4], 2, 10)
    assert list(np.isfinite(got[0])) == [True, True] + [False] * 8


def test_n_cols_truncates():
    got = oracle.index_scores_dense(np.ones((1, 1, 1)), np.ones((1, 1)), np.ones((10, 1)),
                                    [0], [0], [9], 1, 4)
    assert got.shape == (1, 4) and np.all(got == 1.0)


def test_pool_scores_equal_dense_at_pool_positions():
    rng = np.random.default_rng(8)
    q = rng.normal(size=(2, 32, 128))
    w = rng.normal(size=(2, 32))
    k = rng.normal(size=(200, 128))
    q_pos = np.array([99, 60])
    seq_base = [0, 100]
    q_seq = [0, 1]
    dense = oracle.index_scores_dense(q, w, k, seq_base, q_seq, q_pos, 1, 100)
    cand = np.array([[0, 3, 12, -1], [2, 7, -1, -1]])
    pool = oracle.index_scores_pool(q, w, k, seq_base, q_seq, q_pos, 1, cand, 8)
    pos = oracle.pool_positions(cand, 8)
    assert pool.shape == (2, 32)
    for t in range(2):
        for i in range(32):
            p = pos[t, i]
            if p < 0 or p > q_pos[t]:
                assert pool[t, i] == -np.inf
            else:
                assert np.isclose(pool[t, i], dense[t, p], rtol=1e-13, atol=1e-12)
    # block 7 of query 1 holds positions 56..63, of which 56..60 are visible
    assert np.isfinite(pool[1, 8:13]).all() and np.isinf(pool[1, 13:16]).all()
