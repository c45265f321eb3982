"""Pins of the oracle's top-k and block-candidate selection."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rank_select(values, k):
    """Brute force by counting: entry i is chosen iff it is finite and fewer
    than k finite entries beat it (higher value, or equal value at a lower
    position)."""
    n = len(values)
    chosen = []
    for i in range(n):
        if not values[i] > -np.inf:
            continue
        better = sum(1 for j in range(n) if values[j] > -np.inf and
                     (values[j] > values[i] or (values[j] == values[i] and j < i)))
        if better < k:
            chosen.append(i)
    return chosen + [-1] * (k - len(chosen))


def test_topk_golden_ties():
    for case in _gold("topk_ties.json")["cases"]:
        v = np.array([float(x) for x in case["scores"]])
        got = oracle.topk(v, np.arange(len(v)), case["k"])
        assert list(got) == case["expect"], case


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_tie_heavy(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    v = rng.integers(-3, 4, size=n).astype(float)
    v[rng.random(n) < 0.2] = -np.inf
    k = int(rng.integers(1, 20))
    assert list(oracle.topk(v, np.arange(n), k)) == _rank_select(list(v), k)


def test_topk_matches_torch_on_distinct_values():
    x = torch.randn(5000, generator=torch.Generator().manual_seed(4), dtype=torch.float64)
    ref = np.sort(torch.topk(x, 512).indices.numpy())
    got = oracle.topk(x.numpy(), np.arange(5000), 512)
    assert np.array_equal(got, ref)


def test_topk_selects_all_when_short():
    """DSA page, 'design': when S <= k top-k selects every token."""
    v = np.random.default_rng(1).normal(size=300)
    got = oracle.topk(v, np.arange(300), 512)
    assert list(got[:300]) == list(range(300)) and np.all(got[300:] == -1)


def test_topk_positions_follow_given_positions():
    v = np.array([1.0, 5.0, 5.0, 2.0])
    pos = np.array([40, 41, 16, 17])      # ties resolve on the position
    assert list(oracle.topk(v, pos, 2)) == [16, 41]


def test_block_candidates_worked_example():
    g = _gold("blocks_worked_example.json")
    row = np.array(g["row"])
    bm = oracle.block_maxima(row, len(row), g["block_size"])
    assert list(bm[:3]) == g["block_maxima_first_three"]
    pos = np.array([len(row) - 1])
    for keep, key in [(2, "pool_keep_2"), (3, "pool_keep_3")]:
        got = oracle.block_candidates(row[None], pos, 1, 8, keep)[0]
        assert list(got) == g[key]
    mm = g["max_vs_mean"]
    r = np.array(mm["row"])
    got = oracle.block_candidates(r[None], [len(r) - 1], 1, 8, mm["keep"])[0]
    assert list(got) == mm["pool"]
    # the same selection driven by block means would choose differently
    means = r.reshape(-1, 8).mean(1)
    means[-1] = np.inf
    assert list(oracle.topk(means, np.arange(3), 2)) == mm["pool_if_mean_were_used"]


def _brute_blocks(row, n, bs, keep):
    nb = -(-n // bs)
    bm = [max(row[b * bs:min(n, (b + 1) * bs)]) for b in range(nb)]
    bm[-1] = np.inf
    return _rank_select(bm, keep)


@pytest.mark.parametrize("seed", range(6))
def test_block_candidates_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n_cols = 200
    pos = int(rng.integers(0, 200))
    row = rng.integers(-5, 6, size=n_cols).astype(float)
    keep = int(rng.integers(1, 12))
    got = oracle.block_candidates(row[None], [pos], 1, 8, keep)[0]
    assert list(got) == _brute_blocks(row, pos + 1, 8, keep)


def test_block_candidates_invariants():
    """CSA2 page, 'blocks are not compression' (without ties the pool holds
    the Full layer's own top-k) and 'which positions are in the pool' (at
    most n_blocks blocks; every block when there are no more than that; the
    latest block always)."""
    rng = np.random.default_rng(9)
    n = 5000
    row = rng.normal(size=n)
    pool = oracle.block_candidates(row[None], [n - 1], 1, 8, 200)[0]
    assert np.all(pool >= 0) and len(pool) == 200
    assert (n - 1) // 8 in set(pool)
    top = oracle.topk(row, np.arange(n), 150)
    assert set(top // 8) <= set(pool)
    few = oracle.block_candidates(row[None, :1000], [999], 1, 8, 200)[0]
    assert list(few[:125]) == list(range(125)) and np.all(few[125:] == -1)


def test_reindex_pool_topk_equals_masked_dense_topk():
    """CSA2 page, 'where attention is computed': the default path masks the
    dense scores outside the pool to -inf and runs the ordinary top-k; the
    candidate indexer scores only the pool.  Both must choose the same
    positions, and every chosen position lies in the pool."""
    rng = np.random.default_rng(21)
    q = rng.normal(size=(1, 32, 128))
    w = rng.normal(size=(1, 32))
    k = rng.normal(size=(3000, 128))
    dense = oracle.index_scores_dense(q, w, k, [0], [0], [2999], 1, 3000)
    cand = oracle.block_candidates(dense, [2999], 1, 8, 40)
    pool = oracle.index_scores_pool(q, w, k, [0], [0], [2999], 1, cand, 8)
    got = oracle.topk_rows_pool(pool, cand, 8, 64)[0]
    members = oracle.pool_positions(cand, 8)[0]
    masked = np.full(3000, -np.inf)
    masked[members[members >= 0]] = dense[0, members[members >= 0]]
    ref = oracle.topk(masked, np.arange(3000), 64)
    assert np.array_equal(got, ref)
    assert set(got) <= set(members)


def test_reindex_equals_full_when_pool_covers_everything():
    """CSA2 page, 'which positions are in the pool': when the sequence has at
    most n_blocks blocks the pool is every visible position, so pool scoring
    and full scoring pick the same top-k."""
    rng = np.random.default_rng(22)
    q = rng.normal(size=(1, 32, 128))
    w = rng.normal(size=(1, 32))
    k = rng.normal(size=(1000, 128))
    dense = oracle.index_scores_dense(q, w, k, [0], [0], [997], 1, 1000)
    cand = oracle.block_candidates(dense, [997], 1, 8, 2048)
    pool = oracle.index_scores_pool(q, w, k, [0], [0], [997], 1, cand, 8)
    assert np.array_equal(oracle.topk_rows_pool(pool, cand, 8, 512),
                          oracle.topk_rows_dense(dense, [997], 1, 512))
