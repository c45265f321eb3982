"""Parity of the HIP path with the oracle on small inputs that still span
several tiles, chunks and ragged tails.  Every call goes through libcsa2.so."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_long_amd as tsl
from top_sparse_long_amd.driver import LayerRunner
from tests import oracle_io
from tests.parity import (check_scores, check_index_table, check_topk_gap, check_attention,
                          row_tau)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsl.load()


def _np(t):
    return t.detach().cpu().numpy()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# index scores

@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
@pytest.mark.parametrize("ratio", [1, 2])
def test_index_scores_fp8_ragged(ratio, k_fmt):
    n_entries = [5000, 7777, 1, 3, 2049]
    positions = [[n * ratio - 1, n * ratio - 2, 17] for n in n_entries[:2]] + \
                [[ratio - 1], [3 * ratio - 1, 0], [2049 * ratio - 1]]
    _announce(f"index_scores fp8 ratio={ratio} keys={k_fmt}")
    wl = synth.mini_workload(10 + ratio, n_entries, ratio=ratio, positions=positions,
                             k_fmt=k_fmt).to(DEV)
    run = LayerRunner(wl)
    run.index_scores(0, pool=False)
    torch.cuda.synchronize()
    gpu = _np(run.scores[:, :run.n_cols])
    m = oracle_io.meta(wl)
    ref = oracle.index_scores_dense(oracle_io.index_q(wl.layers[0], True),
                                    oracle_io.index_w(wl.layers[0], True),
                                    oracle_io.index_k_rows(wl), m["seq_base"], m["q_seq"],
                                    m["q_pos"], ratio, run.n_cols)
    check_scores(gpu, ref)


def _prefill_positions(n_tok, n_q, seed):
    """n_q causal positions of one sequence of n_tok tokens: the chunk's tail
    plus a few early positions (nearly empty rows)."""
    rng = np.random.default_rng(seed)
    tail = list(range(n_tok - (n_q - 6), n_tok))
    early = sorted(rng.choice(np.arange(0, 64), size=6, replace=False).tolist())
    return early + tail


@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
@pytest.mark.parametrize("case", ["one_sequence", "mixed_tiles", "long_runs"])
def test_index_scores_prefill_fp8(case, k_fmt):
    """Many queries (at least the query-tiled kernel's threshold): a ragged
    count, causal m = 2 rows of different lengths, in the mixed case 16-query
    tiles that straddle sequences, and with long_runs enough work that each
    workgroup streams a run of more than the minimum eight key blocks (83
    blocks in runs of 10, the last one short)."""
    if case == "one_sequence":
        n_entries = [5000]
        positions = [_prefill_positions(10000, 300, 1)]
    elif case == "long_runs":
        n_entries = [21200]
        positions = [_prefill_positions(42400, 512, 9)]
    else:
        n_entries = [3000, 2100, 4100]
        positions = [_prefill_positions(2 * n, nq, 2 + i)
                     for i, (n, nq) in enumerate(zip(n_entries, (101, 90, 83)))]
    _announce(f"index_scores prefill fp8 {case} keys={k_fmt}")
    wl = synth.mini_workload(60, n_entries, ratio=2, positions=positions, k_fmt=k_fmt).to(DEV)
    assert wl.Q >= 256
    run = LayerRunner(wl)
    run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    gpu = _np(run.scores[:, :run.n_cols])
    m = oracle_io.meta(wl)
    ref = oracle.index_scores_dense(oracle_io.index_q(wl.layers[0], True),
                                    oracle_io.index_w(wl.layers[0], True),
                                    oracle_io.index_k_rows(wl), m["seq_base"], m["q_seq"],
                                    m["q_pos"], 2, run.n_cols)
    check_scores(gpu, ref)
    # fused block maxima of the GPU's own scores
    nb = -(-run.n_cols // 8)
    bm = _np(run.block_max[:, :nb]).astype(np.float64)
    nvis = oracle.visible_count(m["q_pos"], 2)
    for t in range(wl.Q):
        refb = oracle.block_maxima(gpu[t].astype(np.float64), int(nvis[t]), 8)
        assert np.array_equal(bm[t, :len(refb)], refb), t
        assert np.all(bm[t, len(refb):] == -np.inf), t


ONE_TILE_MAX_KEYS = 3 << 19      # dense decode calls above this many query x column keys


@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
def test_index_scores_dense_two_tile_ragged(k_fmt):
    """Dense decode calls of more than 1.5M keys (queries x columns) run the
    two-tile-per-wave kernel.  Eight queries over ragged rows of up to
    200,003 columns reach it: partial last sub-chunks, fused block maxima on
    ragged tails, and (paged) page lookups at the rows' ends.  The paged run
    moves the same bytes through other addresses and must equal the flat run
    bit for bit."""
    n_entries = [200003, 150001, 77, 199990]
    positions = [[200002, 123457], [150000, 149999], [76, 3], [199989, 511]]
    _announce(f"index_scores dense two-tile kernel keys={k_fmt}")
    wl = synth.mini_workload(45, n_entries, positions=positions, k_fmt=k_fmt).to(DEV)
    flat = LayerRunner(wl)
    assert wl.Q * flat.n_cols > ONE_TILE_MAX_KEYS
    paged = LayerRunner(wl, paged=synth.paged_layout(wl, 46))
    for run in (flat, paged):
        run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    gpu = _np(flat.scores[:, :flat.n_cols])
    m = oracle_io.meta(wl)
    ref = oracle.index_scores_dense(oracle_io.index_q(wl.layers[0], True),
                                    oracle_io.index_w(wl.layers[0], True),
                                    oracle_io.index_k_rows(wl), m["seq_base"], m["q_seq"],
                                    m["q_pos"], 1, flat.n_cols)
    check_scores(gpu, ref)
    nb = -(-flat.n_cols // 8)
    bm = _np(flat.block_max[:, :nb]).astype(np.float64)
    nvis = oracle.visible_count(m["q_pos"], 1)
    for t in range(wl.Q):
        refb = oracle.block_maxima(gpu[t].astype(np.float64), int(nvis[t]), 8)
        assert np.array_equal(bm[t, :len(refb)], refb), t
        assert np.all(bm[t, len(refb):] == -np.inf), t
    assert torch.equal(flat.scores[:, :flat.n_cols], paged.scores[:, :paged.n_cols])
    assert torch.equal(flat.block_max[:, :nb], paged.block_max[:, :nb])


def test_index_scores_f32_exact():
    _announce("index_scores f32 integer-exact")
    wl = synth.mini_workload(3, [3000, 777], q_per_seq=3, quantized=False).to(DEV)
    run = LayerRunner(wl)
    run.index_scores(0, pool=False)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    ref = oracle.index_scores_dense(oracle_io.index_q(wl.layers[0], False),
                                    oracle_io.index_w(wl.layers[0], False),
                                    oracle_io.index_k_rows(wl), m["seq_base"], m["q_seq"],
                                    m["q_pos"], 1, run.n_cols)
    gpu = _np(run.scores[:, :run.n_cols]).astype(np.float64)
    assert np.array_equal(gpu, ref)


@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
def test_pool_scores_fp8(k_fmt):
    _announce(f"index_scores pool mode keys={k_fmt}")
    wl = synth.mini_workload(4, [9000, 4000], q_per_seq=2, modes=("reindex",),
                             n_blocks=300, k_fmt=k_fmt).to(DEV)
    rng = np.random.default_rng(4)
    Q = wl.Q
    cand = np.full((Q, 300), -1, dtype=np.int32)
    nvis = _np(wl.n_vis())
    for t in range(Q):
        nb = -(-int(nvis[t]) // 8)
        # include blocks past the visible range and the partial last block
        pick = np.sort(rng.choice(nb + 5, size=min(250, nb + 5), replace=False))
        cand[t, :len(pick)] = pick
    run = LayerRunner(wl)
    run.slots.candidates = torch.from_numpy(cand).to(DEV)
    run.index_scores(0, pool=True)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    ref = oracle.index_scores_pool(oracle_io.index_q(wl.layers[0], True),
                                   oracle_io.index_w(wl.layers[0], True),
                                   oracle_io.index_k_rows(wl), m["seq_base"], m["q_seq"],
                                   m["q_pos"], 1, cand, 8)
    check_scores(_np(run.pool_scores[:, :run.pool_cols]), ref, "pool scores")


# ---------------------------------------------------------------------------
# selection: the oracle reads the same fp32 scores, so indices are bit-exact

def _tie_scores(rng, Q, n_cols, levels):
    x = rng.integers(-levels, levels + 1, size=(Q, n_cols)).astype(np.float32)
    return x


@pytest.mark.parametrize("n_cols,k", [(1, 512), (100, 512), (511, 512), (513, 512),
                                      (5000, 512), (32768, 512), (40000, 512),
                                      (131072, 512), (300000, 2048), (1 << 20, 512)])
def test_topk_dense_exact(n_cols, k):
    _announce(f"topk dense n_cols={n_cols} k={k}")
    rng = np.random.default_rng(n_cols)
    Q = 3
    sc = _tie_scores(rng, Q, n_cols, 50 if n_cols > 1000 else 3)
    # visible prefixes: full, ragged, tiny
    q_pos = np.array([n_cols - 1, max(0, (2 * n_cols) // 3 - 1), 0], dtype=np.int32)
    stride = (n_cols + 63) // 64 * 64
    dev = torch.full((Q, stride), float("nan"), device=DEV)
    dev[:, :n_cols] = torch.from_numpy(sc).to(DEV)
    qp = torch.from_numpy(q_pos).to(DEV)
    idx = torch.empty((Q, k), dtype=torch.int32, device=DEV)
    ws = torch.empty((max(16, tsl.csa2_topk_workspace_size(Q, n_cols, k)),), dtype=torch.uint8,
                     device=DEV)
    tsl.csa2_topk(dev, n_cols, qp, 1, k, idx, ws, Q)
    torch.cuda.synchronize()
    ref = oracle.topk_rows_dense(sc.astype(np.float64), q_pos, 1, k)
    assert np.array_equal(_np(idx), ref)


def test_topk_dense_with_neg_inf():
    _announce("topk dense with -inf entries")
    rng = np.random.default_rng(7)
    sc = rng.normal(size=(4, 70000)).astype(np.float32)
    sc[0, :] = -np.inf
    sc[1, rng.random(70000) < 0.995] = -np.inf       # ~350 finite: fewer than k
    sc[2, ::2] = -np.inf
    dev = torch.from_numpy(sc).to(DEV)
    idx = torch.empty((4, 512), dtype=torch.int32, device=DEV)
    ws = torch.empty((tsl.csa2_topk_workspace_size(4, 70000, 512),), dtype=torch.uint8, device=DEV)
    tsl.csa2_topk(dev, 70000, None, 1, 512, idx, ws, 4)
    torch.cuda.synchronize()
    ref = np.stack([oracle.topk(sc[t].astype(np.float64), np.arange(70000), 512) for t in range(4)])
    assert np.array_equal(_np(idx), ref)
    assert np.all(_np(idx)[0] == -1)


def test_topk_pool_exact():
    _announce("topk pool mode")
    rng = np.random.default_rng(8)
    Q, nb, bs = 3, 2048, 8
    cand = np.full((Q, nb), -1, dtype=np.int32)
    for t in range(Q):
        n = [2048, 1500, 10][t]
        cand[t, :n] = np.sort(rng.choice(200000, n, replace=False))
    sc = _tie_scores(rng, Q, nb * bs, 20)
    idx = torch.empty((Q, 512), dtype=torch.int32, device=DEV)
    tsl.csa2_topk(torch.from_numpy(sc).to(DEV), nb * bs, None, 1, 512, idx, None, Q,
                  cand=torch.from_numpy(cand).to(DEV), block_size=bs)
    torch.cuda.synchronize()
    ref = oracle.topk_rows_pool(sc.astype(np.float64), cand, bs, 512)
    assert np.array_equal(_np(idx), ref)


@pytest.mark.parametrize("n_cols,n_blocks", [(100, 16), (16000, 2048), (20000, 2048),
                                             (300000, 2048), (1 << 20, 2048), (50000, 64)])
def test_block_candidates_exact(n_cols, n_blocks):
    _announce(f"block_candidates n_cols={n_cols} n_blocks={n_blocks}")
    rng = np.random.default_rng(n_cols + n_blocks)
    Q = 2
    sc = _tie_scores(rng, Q, n_cols, 40)
    q_pos = np.array([n_cols - 1, max(0, n_cols // 2 - 4)], dtype=np.int32)
    cand = torch.empty((Q, n_blocks), dtype=torch.int32, device=DEV)
    ws = torch.empty((max(16, tsl.csa2_block_candidates_workspace_size(Q, n_cols, 8, n_blocks)),),
                     dtype=torch.uint8, device=DEV)
    tsl.csa2_block_candidates(torch.from_numpy(sc).to(DEV), n_cols,
                              torch.from_numpy(q_pos).to(DEV), 1, 8, n_blocks, cand, ws, Q)
    torch.cuda.synchronize()
    ref = oracle.block_candidates(sc.astype(np.float64), q_pos, 1, 8, n_blocks)
    assert np.array_equal(_np(cand), ref)


@pytest.mark.parametrize("from_block_max", [False, True])
@pytest.mark.parametrize("n_cols,n_blocks,k,ratio", [(100, 16, 512, 1), (20000, 2048, 512, 2),
                                                     (131072, 2048, 512, 1),
                                                     (300000, 2048, 2048, 1),
                                                     (1 << 20, 2048, 512, 2)])
def test_topk_and_block_candidates_exact(n_cols, n_blocks, k, ratio, from_block_max):
    """The shared-launch call gives the oracle's top-k and pool, and the same
    bits as the two separate calls."""
    _announce(f"topk_and_block_candidates n_cols={n_cols} n_blocks={n_blocks} k={k} "
              f"ratio={ratio} block_max={from_block_max}")
    rng = np.random.default_rng(n_cols + k + ratio)
    Q, bs = 3, 8
    sc = _tie_scores(rng, Q, n_cols, 40)
    last = [ratio * n_cols - 1, max(0, (ratio * n_cols) // 3 - 5), 0]
    q_pos = np.array(last, dtype=np.int32)
    nvis = oracle.visible_count(q_pos, ratio)
    stride = (n_cols + 63) // 64 * 64
    dev = torch.full((Q, stride), float("nan"), device=DEV)
    dev[:, :n_cols] = torch.from_numpy(sc).to(DEV)
    bm = None
    if from_block_max:
        nb = -(-n_cols // bs)
        host = np.full((Q, nb), -np.inf)
        for t in range(Q):
            m = oracle.block_maxima(sc[t].astype(np.float64), int(min(nvis[t], n_cols)), bs)
            host[t, :len(m)] = m
        bm = torch.from_numpy(host.astype(np.float32)).to(DEV)
    qp = torch.from_numpy(q_pos).to(DEV)
    idx = torch.empty((Q, k), dtype=torch.int32, device=DEV)
    cand = torch.empty((Q, n_blocks), dtype=torch.int32, device=DEV)
    wsb = tsl.csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, bs, n_blocks)
    ws = torch.randint(0, 255, (max(16, wsb),), dtype=torch.uint8, device=DEV)
    tsl.csa2_topk_and_block_candidates(dev, n_cols, qp, ratio, k, idx, bs, n_blocks, cand, ws, Q,
                                       block_max=bm)
    torch.cuda.synchronize()
    sc64 = sc.astype(np.float64)
    assert np.array_equal(_np(idx), oracle.topk_rows_dense(sc64, q_pos, ratio, k))
    assert np.array_equal(_np(cand), oracle.block_candidates(sc64, q_pos, ratio, bs, n_blocks))
    # the separate calls, bit for bit
    idx2, cand2 = torch.empty_like(idx), torch.empty_like(cand)
    ws_t = torch.empty((max(16, tsl.csa2_topk_workspace_size(Q, n_cols, k)),), dtype=torch.uint8,
                       device=DEV)
    ws_b = torch.empty((max(16, tsl.csa2_block_candidates_workspace_size(Q, n_cols, bs, n_blocks)),),
                       dtype=torch.uint8, device=DEV)
    tsl.csa2_topk(dev, n_cols, qp, ratio, k, idx2, ws_t, Q)
    tsl.csa2_block_candidates(dev, n_cols, qp, ratio, bs, n_blocks, cand2, ws_b, Q, block_max=bm)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cand, cand2)


@pytest.mark.parametrize("n_cols,k,ratio,levels,bs", [(100, 512, 1, 3, 8), (4099, 512, 1, 2, 8),
                                                       (20000, 512, 2, 40, 8), (32768, 512, 2, 40, 8),
                                                       (32768, 512, 2, 1, 8), (131072, 512, 1, 50, 8),
                                                       (200000, 2048, 1, 50, 8),
                                                       (300000, 2048, 1, 50, 8),
                                                       (1 << 20, 512, 1, 60, 8),
                                                       (50000, 512, 1, 30, 32),
                                                       (70000, 2048, 2, 30, 32)])
def test_topk_from_block_max_exact(n_cols, k, ratio, levels, bs):
    """The top-k through the block maxima equals the oracle's dense top-k bit
    for bit, ties included (integer scores with few levels make many blocks
    share their maximum).  The block ranking takes one, two and three
    selection stages; k * block_size above 32,768 takes the dense fallback."""
    _announce(f"topk_from_block_max n_cols={n_cols} k={k} ratio={ratio} levels={levels} bs={bs}")
    rng = np.random.default_rng(n_cols + 3 * k + ratio + levels + bs)
    Q = 4
    sc = _tie_scores(rng, Q, n_cols, levels)
    last = [ratio * n_cols - 1, max(0, (ratio * n_cols) // 3 - 5), ratio * 700 + 1, 0]
    q_pos = np.array(last, dtype=np.int32)
    nvis = oracle.visible_count(q_pos, ratio)
    stride = (n_cols + 63) // 64 * 64
    dev = torch.full((Q, stride), float("nan"), device=DEV)
    dev[:, :n_cols] = torch.from_numpy(sc).to(DEV)
    nb = -(-n_cols // bs)
    host = np.full((Q, nb + 5), np.nan)
    host[:, :nb] = -np.inf
    for t in range(Q):
        m = oracle.block_maxima(sc[t].astype(np.float64), int(min(nvis[t], n_cols)), bs)
        host[t, :len(m)] = m
    bm = torch.from_numpy(host.astype(np.float32)).to(DEV)
    qp = torch.from_numpy(q_pos).to(DEV)
    idx = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    wsb = tsl.csa2_topk_from_block_max_workspace_size(Q, n_cols, k, bs)
    ws = torch.randint(0, 255, (max(16, wsb),), dtype=torch.uint8, device=DEV)
    tsl.csa2_topk_from_block_max(dev, n_cols, bm, qp, ratio, bs, k, idx, ws, Q)
    torch.cuda.synchronize()
    assert np.array_equal(_np(idx), oracle.topk_rows_dense(sc.astype(np.float64), q_pos, ratio, k))


def test_selections_many_rows():
    """Grids of 1,100 rows take the 256-thread selection form for chunks of at
    most 4,096 entries: the dense top-k, the pool top-k, block candidates and
    the top-k through block maxima all equal the oracle bit for bit."""
    _announce("selections over 1,100 rows")
    rng = np.random.default_rng(1100)
    Q, n, bs, k = 1100, 4099, 8, 512
    sc = _tie_scores(rng, Q, n, 20)
    q_pos = rng.integers(0, n + 300, size=Q).astype(np.int32)   # ragged, some rows all visible
    q_pos[:5] = [0, 1, 510, 511, n - 1]
    sc64 = sc.astype(np.float64)
    dev = torch.full((Q, 4160), float("nan"), device=DEV)   # row stride a multiple of 4
    dev[:, :n] = torch.from_numpy(sc).to(DEV)
    qp = torch.from_numpy(q_pos).to(DEV)
    ref = oracle.topk_rows_dense(sc64, q_pos, 1, k)
    # the dense top-k of rows of 4,000 (one 4,096-entry chunk each)
    nd = 4000
    idx = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((max(16, tsl.csa2_topk_workspace_size(Q, nd, k)),), dtype=torch.uint8, device=DEV)
    tsl.csa2_topk(dev, nd, qp, 1, k, idx, ws, Q)
    torch.cuda.synchronize()
    assert np.array_equal(_np(idx), oracle.topk_rows_dense(sc64[:, :nd], q_pos, 1, k))
    # block maxima of the visible prefixes, then the block route
    nb = -(-n // bs)
    nvis = oracle.visible_count(q_pos, 1)
    host = np.full((Q, nb), -np.inf)
    for t in range(Q):
        m = oracle.block_maxima(sc64[t], int(min(nvis[t], n)), bs)
        host[t, :len(m)] = m
    bm = torch.from_numpy(host.astype(np.float32)).to(DEV)
    idx2 = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    ws2 = torch.randint(0, 255, (max(16, tsl.csa2_topk_from_block_max_workspace_size(Q, n, k, bs)),),
                        dtype=torch.uint8, device=DEV)
    tsl.csa2_topk_from_block_max(dev, n, bm, qp, 1, bs, k, idx2, ws2, Q)
    torch.cuda.synchronize()
    assert np.array_equal(_np(idx2), ref)
    # block candidates (256 of at most 513 blocks, latest forced)
    cand = torch.empty((Q, 256), dtype=torch.int32, device=DEV)
    wsb = torch.empty((max(16, tsl.csa2_block_candidates_workspace_size(Q, n, bs, 256)),),
                      dtype=torch.uint8, device=DEV)
    tsl.csa2_block_candidates(dev, n, qp, 1, bs, 256, cand, wsb, Q)
    torch.cuda.synchronize()
    cref = oracle.block_candidates(sc64, q_pos, 1, bs, 256)
    assert np.array_equal(_np(cand), cref)
    # pool top-k over 512 candidate blocks of 8 (4,096 pool entries per row)
    pc = np.full((Q, 512), -1, dtype=np.int32)
    for t in range(Q):
        m = int(rng.integers(0, 513))
        pc[t, :m] = np.sort(rng.choice(100000, m, replace=False))
    psc = _tie_scores(rng, Q, 512 * bs, 20)
    pidx = torch.empty((Q, k), dtype=torch.int32, device=DEV)
    tsl.csa2_topk(torch.from_numpy(psc).to(DEV), 512 * bs, None, 1, k, pidx, None, Q,
                  cand=torch.from_numpy(pc).to(DEV), block_size=bs)
    torch.cuda.synchronize()
    assert np.array_equal(_np(pidx), oracle.topk_rows_pool(psc.astype(np.float64), pc, bs, k))


# ---------------------------------------------------------------------------
# attention: the oracle runs on the same indices

def _attn_case(wl, idx_np, layer=0, window=None, split=True):
    run = LayerRunner(wl)
    if not split:
        run.ws_attn = None      # one workgroup per (query, 16 heads)
    else:
        assert run.ws_attn is not None
    run.slots.topk_idxs = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    if window is not None:
        wl.window = window
    run.attention(layer)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    lay = wl.layers[layer]
    ref, ref_lse = oracle.sparse_attn(oracle_io.attn_q(lay, wl.quantized), oracle_io.main_rows(wl),
                                      m["seq_base"], idx_np, oracle_io.swa_rows(lay, wl.quantized),
                                      m["swa_base"], m["swa_pos0"], None, wl.window, m["q_seq"],
                                      m["q_pos"], _np(lay.sink).astype(np.float64),
                                      wl.softmax_scale, wl.ratio)
    gpu = run.out[layer].float()
    return _np(gpu), _np(run.lse[layer]), ref, ref_lse


def _random_idx(rng, nvis, k, frac_valid=1.0):
    idx = np.full((len(nvis), k), -1, dtype=np.int64)
    for t, n in enumerate(nvis):
        m = min(int(n), int(k * frac_valid))
        idx[t, :m] = np.sort(rng.choice(int(n), m, replace=False))
    return idx


@pytest.mark.parametrize("main_fmt", ["fp4", "fp4s16"])
@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("ratio", [1, 2])
def test_sparse_attn_quant(ratio, split, main_fmt):
    _announce(f"sparse_attn quantized ratio={ratio} split={split} main={main_fmt}")
    wl = synth.mini_workload(20 + ratio, [3000, 700, 200], ratio=ratio,
                             positions=[[3000 * ratio - 1, 1500], [700 * ratio - 1], [5, 0]],
                             main_fmt=main_fmt).to(DEV)
    rng = np.random.default_rng(ratio)
    nvis = _np(wl.n_vis())
    idx = _random_idx(rng, nvis, 512, 0.9)
    idx[0, 5] = -1            # holes inside the table
    idx = np.where(idx >= 0, idx, -1)
    gpu, gl, ref, rl = _attn_case(wl, idx, split=split)
    check_attention(gpu, ref)
    assert np.abs(gl - rl).max() <= 1e-3


def test_sparse_attn_split_workspace_reuse():
    """One attention workspace across calls of different batch shapes: the
    split records hold nothing that outlives a call, so a repeated call is
    bit-identical and a smaller batch in between does not disturb it."""
    _announce("sparse_attn split workspace reused across batch shapes")
    big = synth.mini_workload(34, [3000, 2500, 2000, 1500, 1000, 900]).to(DEV)
    small = synth.mini_workload(35, [4000, 600, 90], q_per_seq=1).to(DEV)
    rb, rs = LayerRunner(big), LayerRunner(small)
    assert rb.ws_attn is not None and rs.ws_attn is not None
    rs.ws_attn = rb.ws_attn
    rng = np.random.default_rng(36)
    ib = _random_idx(rng, _np(big.n_vis()), 512, 0.9)
    isml = _random_idx(rng, _np(small.n_vis()), 512, 0.7)
    rb.slots.topk_idxs = torch.from_numpy(ib.astype(np.int32)).to(DEV)
    rs.slots.topk_idxs = torch.from_numpy(isml.astype(np.int32)).to(DEV)
    rb.attention(0)
    torch.cuda.synchronize()
    first, first_lse = rb.out[0].clone(), rb.lse[0].clone()
    for _ in range(3):
        rs.attention(0)
        rb.attention(0)
    torch.cuda.synchronize()
    assert torch.equal(rb.out[0], first) and torch.equal(rb.lse[0], first_lse)
    for wl, run, idx in ((big, rb, ib), (small, rs, isml)):
        m = oracle_io.meta(wl)
        lay = wl.layers[0]
        ref, _ = oracle.sparse_attn(oracle_io.attn_q(lay, wl.quantized), oracle_io.main_rows(wl),
                                    m["seq_base"], idx, oracle_io.swa_rows(lay, wl.quantized),
                                    m["swa_base"], m["swa_pos0"], None, wl.window, m["q_seq"],
                                    m["q_pos"], _np(lay.sink).astype(np.float64),
                                    wl.softmax_scale, wl.ratio)
        check_attention(_np(run.out[0].float()), ref)


@pytest.mark.parametrize("split", [True, False])
def test_sparse_attn_ragged_k_and_window(split):
    """A top-k count and a window that are not multiples of the 16-key tile:
    the last main and SWA tiles are partial."""
    _announce(f"sparse_attn ragged k=77 window=50 split={split}")
    wl = synth.mini_workload(37, [3000, 900, 400], topk=77,
                             positions=[[2999, 1200], [899], [399, 30]]).to(DEV)
    rng = np.random.default_rng(38)
    idx = _random_idx(rng, _np(wl.n_vis()), 77, 0.95)
    gpu, gl, ref, rl = _attn_case(wl, idx, window=50, split=split)
    check_attention(gpu, ref)
    assert np.abs(gl - rl).max() <= 1e-3


@pytest.mark.parametrize("split", [True, False])
def test_sparse_attn_largest_k(split):
    """The largest top-k the kernel stages (2048 indices per query)."""
    _announce(f"sparse_attn k=2048 split={split}")
    wl = synth.mini_workload(39, [6000, 2500], q_per_seq=2, topk=2048).to(DEV)
    rng = np.random.default_rng(40)
    idx = _random_idx(rng, _np(wl.n_vis()), 2048, 1.0)
    gpu, gl, ref, rl = _attn_case(wl, idx, split=split)
    check_attention(gpu, ref)
    assert np.abs(gl - rl).max() <= 1e-3


@pytest.mark.parametrize("H,split,q_per_seq", [(16, True, 2), (16, False, 2), (128, True, 1), (128, False, 2),
                                               (128, True, 10), (64, True, 20), (16, True, 150)])
def test_sparse_attn_head_counts(H, split, q_per_seq):
    """Head counts other than 64 (one and eight 16-head groups per query),
    through the C ABI with random bf16 queries and sinks over a workload's
    caches.  The batch sizes reach every launch shape of the 16-head kernel:
    four column parts with the keys split (4 and 16 groups of 16 heads) and
    without (32), two column parts (160 groups) and whole rows (300)."""
    _announce(f"sparse_attn H={H} split={split} queries={2 * q_per_seq}")
    wl = synth.mini_workload(41, [2000, 700], q_per_seq=q_per_seq).to(DEV)
    run = LayerRunner(wl)
    rng = np.random.default_rng(42)
    q = torch.from_numpy(rng.standard_normal((wl.Q, H, 512)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(DEV)
    idx_np = _random_idx(rng, _np(wl.n_vis()), 512, 0.9)
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    out = torch.empty((wl.Q, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((wl.Q, H), dtype=torch.float32, device=DEV)
    ws = None
    nb = tsl.csa2_sparse_attn_workspace_size(wl.Q, H, 512, wl.window)
    # below 128 workgroups (16-head groups x 4 column parts) the keys are split
    assert (nb > 0) == (wl.Q * (H // 16) * 4 < 128)
    if split and nb > 0:
        ws = torch.zeros((nb,), dtype=torch.uint8, device=DEV)
    tsl.csa2_sparse_attn(q, tsl.CSA2_BF16, run.slots.compress_kv, wl.seq_base, idx, 512,
                         run.layer_rows[0]["swa"], wl.swa_base, wl.swa_pos0, None, wl.window,
                         wl.q_seq, wl.q_pos, wl.ratio, sink, wl.softmax_scale, out, tsl.CSA2_BF16,
                         lse, wl.Q, H=H, workspace=ws)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    ref, ref_lse = oracle.sparse_attn(_np(q.float()).astype(np.float64), oracle_io.main_rows(wl),
                                      m["seq_base"], idx_np, oracle_io.swa_rows(wl.layers[0], True),
                                      m["swa_base"], m["swa_pos0"], None, wl.window, m["q_seq"],
                                      m["q_pos"], _np(sink).astype(np.float64), wl.softmax_scale,
                                      wl.ratio)
    check_attention(_np(out.float()), ref)
    assert np.abs(_np(lse) - ref_lse).max() <= 1e-3


def test_sparse_attn_quant_duplicates_and_out_of_range():
    _announce("sparse_attn quantized duplicates / out-of-range indices")
    wl = synth.mini_workload(31, [1000], q_per_seq=2).to(DEV)
    idx = np.full((2, 512), -1, dtype=np.int64)
    idx[0, :130] = np.arange(870, 1000)        # the window positions again (main rows)
    idx[1, :10] = np.arange(10)
    idx[1, 10:20] = 5000                       # beyond the visible count: skipped
    gpu, gl, ref, rl = _attn_case(wl, idx)
    check_attention(gpu, ref)


def test_sparse_attn_empty_key_set():
    _announce("sparse_attn empty key set")
    wl = synth.mini_workload(32, [64], q_per_seq=1).to(DEV)
    idx = np.full((1, 512), -1, dtype=np.int64)
    gpu, gl, ref, rl = _attn_case(wl, idx, window=0)
    assert np.all(gpu == 0)
    assert np.allclose(gl[0], _np(wl.layers[0].sink), atol=1e-6)


@pytest.mark.parametrize("quantized,main_fmt,split", [(True, "fp4", True), (True, "fp4", False),
                                                     (True, "fp4s16", True), (True, "fp4s16", False),
                                                     (False, "fp4", False)])
def test_sparse_attn_bounded_replay_window(quantized, main_fmt, split):
    """CSA2 page, 'CED' (bounded replay): the query at p sees the SWA keys of
    [max(s, p-W+1), p] for the replay start s (swa_lo), and none before the
    oldest stored row (swa_pos0).  Five sequences mix the cases: s inside the
    window, s = p (the current token only), s = p + 1 (no SWA key), stored
    rows that start after p - W + 1, and the whole window."""
    _announce(f"sparse_attn swa_lo/swa_pos0 quantized={quantized} main={main_fmt} split={split}")
    n_entries = [3000, 1500, 900, 2600, 700]
    wl = synth.mini_workload(43, n_entries, quantized=quantized, main_fmt=main_fmt).to(DEV)
    run = LayerRunner(wl)
    if not split:
        run.ws_attn = None
    else:
        assert run.ws_attn is not None
    q_pos = _np(wl.q_pos).astype(np.int64)
    lo = np.zeros(5, dtype=np.int64)
    lo[0] = q_pos[0] - 60
    lo[1] = q_pos[1]
    lo[2] = q_pos[2] + 1
    # sequence 3 holds only its last 88 SWA rows: the same rows, with the
    # oldest stored position moved up by 40
    pos0 = _np(wl.swa_pos0).astype(np.int64)
    base = _np(wl.swa_base).astype(np.int64)
    assert pos0[3] == q_pos[3] - wl.window + 1
    pos0[3] += 40
    base[3] += 40
    swa_lo = torch.from_numpy(lo.astype(np.int32)).to(DEV)
    swa_pos0 = torch.from_numpy(pos0.astype(np.int32)).to(DEV)
    swa_base = torch.from_numpy(base).to(DEV)
    rng = np.random.default_rng(44)
    idx_np = _random_idx(rng, _np(wl.n_vis()), 512, 0.9)
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    lay = wl.layers[0]
    dt = tsl.CSA2_BF16 if quantized else tsl.CSA2_F32
    tsl.csa2_sparse_attn(lay.q, dt, run.slots.compress_kv, wl.seq_base, idx, 512,
                         run.layer_rows[0]["swa"], swa_base, swa_pos0, swa_lo, wl.window,
                         wl.q_seq, wl.q_pos, wl.ratio, lay.sink, wl.softmax_scale, run.out[0], dt,
                         run.lse[0], wl.Q, workspace=run.ws_attn)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    ref, ref_lse = oracle.sparse_attn(oracle_io.attn_q(lay, quantized), oracle_io.main_rows(wl),
                                      m["seq_base"], idx_np, oracle_io.swa_rows(lay, quantized),
                                      base, pos0, lo, wl.window, m["q_seq"], m["q_pos"],
                                      _np(lay.sink).astype(np.float64), wl.softmax_scale, wl.ratio)
    n_swa = [oracle.attention_keys(t, oracle_io.main_rows(wl), m["seq_base"], np.full((5, 1), -1),
                                   oracle_io.swa_rows(lay, quantized), base, pos0, lo, wl.window,
                                   m["q_seq"], m["q_pos"]).shape[0] for t in range(5)]
    assert n_swa == [61, 1, 0, 88, 128]
    gpu = _np(run.out[0].float())
    check_attention(gpu, ref)
    assert np.abs(_np(run.lse[0]) - ref_lse).max() <= 1e-3
    # the unbounded call differs exactly on the bounded sequences
    full, _ = oracle.sparse_attn(oracle_io.attn_q(lay, quantized), oracle_io.main_rows(wl),
                                 m["seq_base"], idx_np, oracle_io.swa_rows(lay, quantized),
                                 m["swa_base"], m["swa_pos0"], None, wl.window, m["q_seq"],
                                 m["q_pos"], _np(lay.sink).astype(np.float64), wl.softmax_scale,
                                 wl.ratio)
    assert np.array_equal(full[4], ref[4])
    for t in range(4):
        assert np.abs(full[t] - ref[t]).max() > 1e-2, t


WIDE_MIN_Q = 256     # 64-head batches of at least this many queries run one workgroup per query


@pytest.mark.parametrize("case", ["fp4_rope_holes", "fp4s16_m2_ragged", "fp4_bounded_window"])
def test_sparse_attn_wide_batch(case):
    """Batches of at least 256 queries with 64 heads run the wide form (all
    heads of a query in one workgroup, rounds of 128 keys, P V from the raw
    codes through transposing LDS reads).  Three hundred queries over ragged
    caches: holes, duplicates and indices past the visible count; the inverse
    RoPE of the output; the pages' 288-byte records at m = 2 with a top-k
    count and window that leave partial tiles and rounds; and the
    bounded-replay window (CSA2 page, CED section)."""
    _announce(f"sparse_attn wide batch {case}")
    ratio = 2 if case == "fp4s16_m2_ragged" else 1
    main_fmt = "fp4s16" if case == "fp4s16_m2_ragged" else "fp4"
    topk = 77 if case == "fp4s16_m2_ragged" else 512
    wl = synth.mini_workload(47, [3000, 1700, 900], q_per_seq=100, ratio=ratio, main_fmt=main_fmt,
                             topk=topk).to(DEV)
    assert wl.Q >= WIDE_MIN_Q
    window = 50 if case == "fp4s16_m2_ragged" else wl.window
    rope = synth.rope_table(3000 * ratio, DEV) if case == "fp4_rope_holes" else None
    run = LayerRunner(wl, rope_cs=rope)
    rng = np.random.default_rng(48)
    idx = _random_idx(rng, _np(wl.n_vis()), topk, 0.95)
    if case == "fp4_rope_holes":
        idx[0, 5] = -1
        idx[1, :130] = np.arange(870, 1000)       # duplicates of window positions
        idx[2, 10:20] = 10 ** 6                   # past the visible count
        idx[3, :] = -1                            # only the window
    q_pos = _np(wl.q_pos).astype(np.int64)
    pos0 = _np(wl.swa_pos0).astype(np.int64)
    base = _np(wl.swa_base).astype(np.int64)
    lo = None
    if case == "fp4_bounded_window":
        q_seq = _np(wl.q_seq)
        lo = np.zeros(wl.B, dtype=np.int64)
        lo[0] = q_pos[q_seq == 0].max() - 60      # inside the window of the sequence's last query
        lo[1] = q_pos[q_seq == 1].max() + 1       # past every query of the sequence: no SWA key
    lo_t = None if lo is None else torch.from_numpy(lo.astype(np.int32)).to(DEV)
    idx_t = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    lay = wl.layers[0]
    tsl.csa2_sparse_attn(lay.q, tsl.CSA2_BF16, run.slots.compress_kv, wl.seq_base, idx_t, topk,
                         run.layer_rows[0]["swa"], wl.swa_base, wl.swa_pos0, lo_t, window, wl.q_seq,
                         wl.q_pos, wl.ratio, lay.sink, wl.softmax_scale, run.out[0], tsl.CSA2_BF16,
                         run.lse[0], wl.Q, workspace=run.ws_attn, rope_cs=rope)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    ref, ref_lse = oracle.sparse_attn(oracle_io.attn_q(lay, True), oracle_io.main_rows(wl),
                                      m["seq_base"], idx, oracle_io.swa_rows(lay, True), base, pos0,
                                      lo, window, m["q_seq"], m["q_pos"],
                                      _np(lay.sink).astype(np.float64), wl.softmax_scale, wl.ratio)
    if rope is not None:
        r = _np(rope).astype(np.float64)
        ref = oracle.unturn_heads(ref, m["q_pos"], r[:, :32], r[:, 32:])
    check_attention(_np(run.out[0].float()), ref)
    assert np.abs(_np(run.lse[0]) - ref_lse).max() <= 1e-3


def test_sparse_attn_f32():
    _announce("sparse_attn f32")
    wl = synth.mini_workload(33, [2048], q_per_seq=4, quantized=False).to(DEV)
    idx = _random_idx(np.random.default_rng(3), _np(wl.n_vis()), 512)
    gpu, gl, ref, rl = _attn_case(wl, idx)
    check_attention(gpu, ref)
    assert np.abs(gpu - ref).max() < 1e-5
    assert np.abs(gl - rl).max() < 1e-5


# ---------------------------------------------------------------------------
# a decoder group end to end, stage by stage

def test_group_end_to_end():
    _announce("group full/reuse/reindex/reuse")
    wl = synth.mini_workload(40, [6000, 3333], q_per_seq=2,
                             modes=("full", "reuse", "reindex", "reuse"),
                             topk=128, n_blocks=60).to(DEV)
    run = LayerRunner(wl)
    m = oracle_io.meta(wl)
    kr = oracle_io.index_k_rows(wl)
    main = oracle_io.main_rows(wl)
    # L0 Full
    run.index_scores(0, pool=False)
    run.block_candidates()
    run.topk(0, pool=False)
    run.attention(0)
    torch.cuda.synchronize()
    l0 = wl.layers[0]
    q0, w0 = oracle_io.index_q(l0, True), oracle_io.index_w(l0, True)
    ref_sc = oracle.index_scores_dense(q0, w0, kr, m["seq_base"], m["q_seq"], m["q_pos"], 1,
                                       run.n_cols)
    gsc = _np(run.scores[:, :run.n_cols])
    check_scores(gsc, ref_sc)
    gsc64 = gsc.astype(np.float64)
    cand = _np(run.cand)
    assert np.array_equal(cand, oracle.block_candidates(gsc64, m["q_pos"], 1, 8, 60))
    idx0 = _np(run.idx[0])
    assert np.array_equal(idx0, oracle.topk_rows_dense(gsc64, m["q_pos"], 1, 128))
    check_index_table(idx0, 128)
    nvis = oracle.visible_count(m["q_pos"], 1)
    for t in range(wl.Q):
        n = int(nvis[t])
        check_topk_gap(idx0[t], ref_sc[t, :n], np.arange(n), 128, row_tau(ref_sc[t]))
    # L1 Reuse reads the same indices
    run.attention(1)
    # L2 Reindex
    run.index_scores(2, pool=True)
    run.topk(2, pool=True)
    run.attention(2)
    run.attention(3)
    torch.cuda.synchronize()
    l2 = wl.layers[2]
    ref_pool = oracle.index_scores_pool(oracle_io.index_q(l2, True), oracle_io.index_w(l2, True),
                                        kr, m["seq_base"], m["q_seq"], m["q_pos"], 1, cand, 8)
    gpool = _np(run.pool_scores[:, :run.pool_cols])
    check_scores(gpool, ref_pool, "pool scores")
    idx2 = _np(run.idx[2])
    assert np.array_equal(idx2, oracle.topk_rows_pool(gpool.astype(np.float64), cand, 8, 128))
    members = oracle.pool_positions(cand, 8)
    for t in range(wl.Q):
        assert set(idx2[t][idx2[t] >= 0]) <= set(members[t][members[t] >= 0])
    for li, idx in [(0, idx0), (1, idx0), (2, idx2), (3, idx2)]:
        lay = wl.layers[li]
        ref, _ = oracle.sparse_attn(oracle_io.attn_q(lay, True), main, m["seq_base"], idx,
                                    oracle_io.swa_rows(lay, True), m["swa_base"], m["swa_pos0"],
                                    None, wl.window, m["q_seq"], m["q_pos"],
                                    _np(lay.sink).astype(np.float64), wl.softmax_scale, 1)
        check_attention(_np(run.out[li].float()), ref, f"layer {li}")


def test_repeat_runs_are_bitwise_identical():
    _announce("determinism")
    wl = synth.mini_workload(41, [70000, 5000], q_per_seq=2, modes=("full", "reindex")).to(DEV)
    run = LayerRunner(wl)
    run.run()
    torch.cuda.synchronize()
    first = [o.clone() for o in run.out] + [run.idx[0].clone(), run.idx[1].clone(), run.cand.clone()]
    run.run()
    torch.cuda.synchronize()
    second = list(run.out) + [run.idx[0], run.idx[1], run.cand]
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_fused_block_max_matches_scores():
    _announce("fused block maxima")
    wl = synth.mini_workload(42, [50000, 9001], q_per_seq=2, modes=("full", "reindex"),
                             positions=[[49999, 30000], [9000, 77]]).to(DEV)
    run = LayerRunner(wl)
    run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    g = _np(run.scores[:, :run.n_cols]).astype(np.float64)
    nb = -(-run.n_cols // 8)
    bm = _np(run.block_max[:, :nb]).astype(np.float64)
    nvis = oracle.visible_count(_np(wl.q_pos), 1)
    for t in range(wl.Q):
        n = int(nvis[t])
        ref = oracle.block_maxima(g[t], n, 8)
        assert np.array_equal(bm[t, :len(ref)], ref)
        assert np.all(bm[t, len(ref):] == -np.inf)
    run.block_candidates(from_block_max=True)
    torch.cuda.synchronize()
    a = _np(run.cand).copy()
    run.block_candidates(from_block_max=False)
    torch.cuda.synchronize()
    assert np.array_equal(a, _np(run.cand))
    assert np.array_equal(a, oracle.block_candidates(g, _np(wl.q_pos), 1, 8, wl.n_blocks))


@pytest.mark.parametrize("many", [False, True])
@pytest.mark.parametrize("bs", [1, 2, 4, 16, 32])
def test_fused_block_max_sizes(bs, many):
    """Block maxima fused into scoring for every supported block size, on the
    per-query kernel and on the query-tiled one (many queries)."""
    _announce(f"fused block maxima bs={bs} many={many}")
    if many:
        wl = synth.mini_workload(44, [3333], ratio=2, block_size=bs,
                                 positions=[_prefill_positions(6666, 260, 7)]).to(DEV)
    else:
        wl = synth.mini_workload(44, [7000, 333], q_per_seq=2, block_size=bs,
                                 positions=[[6999, 4000], [332, 5]]).to(DEV)
    run = LayerRunner(wl)
    run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    g = _np(run.scores[:, :run.n_cols]).astype(np.float64)
    nb = -(-run.n_cols // bs)
    bm = _np(run.block_max[:, :nb]).astype(np.float64)
    nvis = oracle.visible_count(_np(wl.q_pos), wl.ratio)
    for t in range(wl.Q):
        ref = oracle.block_maxima(g[t], int(nvis[t]), bs)
        assert np.array_equal(bm[t, :len(ref)], ref), t
        assert np.all(bm[t, len(ref):] == -np.inf), t


@pytest.mark.parametrize("big", [False, True])
@pytest.mark.parametrize("bs", [8, 32])
def test_block_max_without_scores(bs, big):
    """Dense scoring that writes only the block maxima (the decode kernel
    with a storing wave) gives the maxima of the call that also writes the
    scores, bit for bit: on the one-tile kernel and on the two-tile one
    (above 1.5M keys), with ragged row ends and a query that sees nothing
    (position 0 at m = 2), whose maxima are all -inf."""
    _announce(f"block maxima without scores bs={bs} big={big}")
    n = [900_003, 700_001] if big else [50_001, 9_001]
    pos = [[2 * n[0] - 1, 0], [2 * n[1] - 1 - 999, 2 * 5_000 + 1]]
    wl = synth.mini_workload(45, n, q_per_seq=2, ratio=2, block_size=bs, positions=pos).to(DEV)
    run = LayerRunner(wl)
    run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    nb = -(-run.n_cols // bs)
    ref = run.block_max[:, :nb].clone()
    g = _np(run.scores[:, :run.n_cols]).astype(np.float64)
    run.block_max.fill_(7.0)
    run.index_scores(0, pool=False, block_max=True, scores=False)
    torch.cuda.synchronize()
    assert torch.equal(run.block_max[:, :nb], ref)
    nvis = oracle.visible_count(_np(wl.q_pos), 2)
    assert int(nvis.min()) == 0
    refn = _np(ref).astype(np.float64)
    for t in range(wl.Q):
        r = oracle.block_maxima(g[t], int(nvis[t]), bs)
        assert np.array_equal(refn[t, :len(r)], r), t
        assert np.all(refn[t, len(r):] == -np.inf), t


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
def test_block_max_without_scores_formats(k_fmt, paged):
    """The maxima-only call (the storing-wave form) with FP4 keys and their
    E4M3 scales, and with index keys read through a page table: the same
    block maxima as the score-writing call on the same runner, bit for bit."""
    _announce(f"block maxima without scores keys={k_fmt} paged={paged}")
    n = [300_001, 40_000]
    pos = [[n[0] - 1, 123_457], [n[1] - 1, 0]]
    wl = synth.mini_workload(46, n, q_per_seq=2, positions=pos, k_fmt=k_fmt).to(DEV)
    run = LayerRunner(wl, paged=synth.paged_layout(wl, 76)) if paged else LayerRunner(wl)
    run.index_scores(0, pool=False, block_max=True)
    torch.cuda.synchronize()
    nb = -(-run.n_cols // wl.block_size)
    ref = run.block_max[:, :nb].clone()
    run.block_max.fill_(7.0)
    run.index_scores(0, pool=False, block_max=True, scores=False)
    torch.cuda.synchronize()
    assert torch.equal(run.block_max[:, :nb], ref)
    assert bool(torch.isfinite(ref).any())


@pytest.mark.parametrize("concurrent,n_seq,rescore", [(False, 2, None), (True, 2, None), (True, 4, None),
                                                     (True, 2, True)])
def test_graph_replay_matches_eager(concurrent, n_seq, rescore):
    """A captured pass (optionally with every attention call on a second
    stream, overlapping the later layers' scoring and selection) replays to
    the serial eager result, several times, with eager work and
    synchronisations between the replays.  Overlapped, the Full layer's
    top-k (through its block maxima, or on the re-scoring route) and its
    attention run on the second stream while the main stream ranks the pool
    and scores it; the eager reference is the serial default pass.  With 8
    queries attention splits no keys (no shared workspace)."""
    _announce(f"graph replay concurrent={concurrent} sequences={n_seq} rescore={rescore}")
    wl = synth.mini_workload(43, [70000, 20000, 30000, 5000][:n_seq], q_per_seq=2,
                             modes=("full", "reuse", "reindex")).to(DEV)
    run = LayerRunner(wl, rescore=rescore)
    names = [n for n, _ in run.steps(concurrent=concurrent)]
    side = "topk_top_and_sparse_attn" if rescore else "topk_blocks_and_sparse_attn"
    assert (side in names) == concurrent
    assert (run.ws_attn is None) == (n_seq == 4)
    assert ("topk_and_blocks" in [n for n, _ in run.steps()]) == (not rescore)
    run.run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in run.out] + [run.cand.clone()] + [v.clone() for v in run.idx.values()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.run(concurrent=concurrent)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in run.steps(concurrent=concurrent):
            fn()
    for rep in range(4):
        for o in run.out:
            o.zero_()
        run.cand.fill_(-7)
        for v in run.idx.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(run.out) + [run.cand] + list(run.idx.values())
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
        run.run()              # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
def test_full_layer_rescore_route_equals_dense_route(k_fmt):
    """A Full layer that writes only its block maxima, ranks its best blocks
    (csa2_top_blocks_and_block_candidates) and takes its top-k among their
    keys scored again gives exactly the dense route's top-k, pool and
    attention: the re-scored keys carry the dense scores bit for bit, and the
    k best entries lie in the k best blocks.  Ragged sequences, one shorter
    than k keys, and ratio 2."""
    _announce(f"Full-layer re-scoring route {k_fmt}")
    for ratio in (1, 2):
        wl = synth.mini_workload(91 + ratio, [9000, 3000, 300], q_per_seq=2, ratio=ratio,
                                 modes=("full", "reindex"), k_fmt=k_fmt).to(DEV)
        dense = LayerRunner(wl, rescore=False)
        top = LayerRunner(wl, rescore=True)
        assert top.rescore and not dense.rescore
        dense.run()
        top.run()
        torch.cuda.synchronize()
        assert "index_scores_top" in [n for n, _ in top.steps()]
        for li in dense.idx:
            assert torch.equal(dense.idx[li], top.idx[li]), (ratio, li)
        assert torch.equal(dense.cand, top.cand)
        for a, b in zip(dense.out, top.out):
            assert torch.equal(a, b)
        # the best blocks' re-scored keys equal the dense scores at their columns
        bs = wl.block_size
        tb = _np(top.top_blocks)
        ts = _np(top.top_scores[:, :top.top_cols])
        ds = _np(dense.scores[:, :dense.n_cols])
        for t in range(wl.Q):
            for i, blk in enumerate(tb[t]):
                if blk < 0:
                    assert np.all(ts[t, i * bs:(i + 1) * bs] == -np.inf)
                    continue
                cols = np.arange(blk * bs, min((blk + 1) * bs, dense.n_cols))
                assert np.array_equal(ts[t, i * bs:i * bs + len(cols)], ds[t, cols]), (ratio, t, blk)
        # the best blocks are the k best by maximum, ascending
        bm = _np(dense.block_max)
        nvis = oracle.visible_count(_np(wl.q_pos), wl.ratio)
        for t in range(wl.Q):
            nb = -(-int(nvis[t]) // bs)
            m = bm[t, :nb].astype(np.float64)
            order = sorted(range(nb), key=lambda j: (-m[j], j))
            want = sorted(j for j in order[:wl.topk] if m[j] > -np.inf)
            got = [int(x) for x in tb[t] if x >= 0]
            assert got == want, (ratio, t)
