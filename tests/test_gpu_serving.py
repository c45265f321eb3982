"""GPU parity of the serving-shaped I/O: paged index keys read through a page
table, the top-k writing physical slots, attention gathering by slot, and the
output's inverse RoPE (DSA page, top-k section and implementation notes;
CSA2 page, core formula).

A paged run moves the same bytes through other addresses, so it must equal
the flat run bit for bit (slots being the flat positions translated by the
oracle's slots_from_positions).  The inverse RoPE is checked against the
oracle's attention followed by its unturn_heads, to the attention bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_long_amd as tsl
from top_sparse_long_amd.driver import LayerRunner
from tests import oracle_io
from tests.parity import check_attention

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


def _random_idx(rng, nvis, k, frac_valid=1.0):
    idx = np.full((len(nvis), k), -1, dtype=np.int64)
    for t, n in enumerate(nvis):
        m = min(int(n), int(k * frac_valid))
        idx[t, :m] = np.sort(rng.choice(int(n), m, replace=False))
    return idx


# ---------------------------------------------------------------------------
# inverse RoPE of the attention output

@pytest.mark.parametrize("quantized,split,main_fmt", [(True, True, "fp4"), (True, False, "fp4"),
                                                     (True, True, "fp4s16"), (True, False, "fp4s16"),
                                                     (False, False, "fp4")])
def test_attention_output_is_turned_back(quantized, split, main_fmt):
    _announce(f"attention inverse RoPE quantized={quantized} split={split} main={main_fmt}")
    wl = synth.mini_workload(70, [3000, 700, 200], ratio=1,
                             positions=[[2999, 1500], [699], [150, 0]],
                             quantized=quantized, main_fmt=main_fmt).to(DEV)
    rope = synth.rope_table(3000, DEV)
    run = LayerRunner(wl, rope_cs=rope)
    if not split:
        run.ws_attn = None
    rng = np.random.default_rng(71)
    idx = _random_idx(rng, _np(wl.n_vis()), 512, 0.9)
    run.slots.topk_idxs = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    run.attention(0)
    torch.cuda.synchronize()
    m = oracle_io.meta(wl)
    lay = wl.layers[0]
    ref, _ = oracle.sparse_attn(oracle_io.attn_q(lay, wl.quantized), oracle_io.main_rows(wl),
                                m["seq_base"], idx, oracle_io.swa_rows(lay, wl.quantized),
                                m["swa_base"], m["swa_pos0"], None, wl.window, m["q_seq"],
                                m["q_pos"], _np(lay.sink).astype(np.float64), wl.softmax_scale,
                                wl.ratio)
    r = _np(rope).astype(np.float64)
    ref = oracle.unturn_heads(ref, m["q_pos"], r[:, :32], r[:, 32:])
    gpu = _np(run.out[0].float())
    check_attention(gpu, ref)
    # the unturned dims are untouched by the table
    run2 = LayerRunner(wl)
    if not split:
        run2.ws_attn = None
    run2.slots.topk_idxs = run.slots.topk_idxs
    run2.attention(0)
    torch.cuda.synchronize()
    assert torch.equal(run2.out[0][..., :448], run.out[0][..., :448])
    # a query at position 0 has cos 1, sin 0: nothing turns
    q0 = int(np.where(m["q_pos"] == 0)[0][0])
    assert torch.equal(run2.out[0][q0], run.out[0][q0])


# ---------------------------------------------------------------------------
# top-k written as slots

def test_topk_writes_slots():
    _announce("top-k with a page table (dense, pool, shared launch)")
    wl = synth.mini_workload(72, [20000, 9000], q_per_seq=3, modes=("full", "reindex"),
                             topk=256, n_blocks=200).to(DEV)
    B = wl.B
    width = (max(wl.n_entries) + 63) // 64
    rng = np.random.default_rng(73)
    table_np = rng.permutation(B * width + 5)[:B * width].reshape(B, width).astype(np.int32)
    flat = LayerRunner(wl)
    flat.index_scores(0, pool=False, block_max=True)
    flat.topk_and_blocks(0, from_block_max=True)
    torch.cuda.synchronize()
    q_seq = _np(wl.q_seq)
    # take out the pages of one chosen position of each sequence
    fidx = _np(flat.idx[0])
    for b in range(B):
        t = int(np.where(q_seq == b)[0][0])
        table_np[b, int(fidx[t, 5]) // 64] = -1
    table = torch.from_numpy(table_np).to(DEV)
    paged = LayerRunner(wl)
    paged.pages_topk = tsl.pages_of(table, q_seq=wl.q_seq)
    paged.index_scores(0, pool=False, block_max=True)
    paged.topk_and_blocks(0, from_block_max=True)
    torch.cuda.synchronize()
    want = oracle.slots_from_positions(fidx, q_seq, table_np)
    assert np.array_equal(_np(paged.idx[0]), want)
    assert np.array_equal(_np(paged.cand), _np(flat.cand))     # the pool stays block ids
    assert (want == -1).sum() > (fidx == -1).sum()              # the missing pages showed up
    for run in (flat, paged):
        run.topk(0, pool=False)
        run.index_scores(1, pool=True)
        run.topk(1, pool=True)
        torch.cuda.synchronize()
    assert np.array_equal(_np(paged.idx[0]),
                          oracle.slots_from_positions(_np(flat.idx[0]), q_seq, table_np))
    assert np.array_equal(_np(paged.idx[1]),
                          oracle.slots_from_positions(_np(flat.idx[1]), q_seq, table_np))


# ---------------------------------------------------------------------------
# paged index keys

def _paged_pair(wl, seed):
    pl = synth.paged_layout(wl, seed)
    return LayerRunner(wl), LayerRunner(wl, paged=pl), pl


@pytest.mark.parametrize("k_fmt", ["fp8", "fp4s16"])
def test_paged_scores_equal_flat(k_fmt):
    _announce(f"paged index scores, keys {k_fmt}")
    wl = synth.mini_workload(74, [5000, 700, 130], ratio=2,
                             positions=[[9999, 4000], [1399], [259, 7]], k_fmt=k_fmt,
                             modes=("full", "reindex"), topk=128, n_blocks=60).to(DEV)
    flat, paged, pl = _paged_pair(wl, 75)
    for run in (flat, paged):
        run.index_scores(0, pool=False, block_max=True)
        run.block_candidates(from_block_max=True)
        run.index_scores(1, pool=True)
        torch.cuda.synchronize()
    nbm = (flat.n_cols + wl.block_size - 1) // wl.block_size
    assert torch.equal(flat.scores[:, :flat.n_cols], paged.scores[:, :paged.n_cols])
    assert torch.equal(flat.block_max[:, :nbm], paged.block_max[:, :nbm])
    assert torch.equal(flat.pool_scores[:, :flat.pool_cols], paged.pool_scores[:, :paged.pool_cols])
    # a page taken out of the table: its positions score -inf, nothing else moves
    pl.page_table[0, 2] = -1
    paged.index_scores(0, pool=False)
    torch.cuda.synchronize()
    f, g = _np(flat.scores), _np(paged.scores)
    q_seq = _np(wl.q_seq)
    for t in range(wl.Q):
        hole = np.zeros(flat.n_cols, dtype=bool)
        if q_seq[t] == 0:
            hole[128:192] = True
        assert np.all(g[t, :flat.n_cols][hole] == -np.inf)
        assert np.array_equal(g[t, :flat.n_cols][~hole], f[t, :flat.n_cols][~hole])


def test_paged_prefill_scores_equal_flat():
    _announce("paged index scores, query-tiled kernel")
    pos = list(range(3000, 3300))
    wl = synth.mini_workload(76, [3300], positions=[pos]).to(DEV)
    assert wl.Q >= 256
    flat, paged, pl = _paged_pair(wl, 77)
    for run in (flat, paged):
        run.index_scores(0, pool=False)
        torch.cuda.synchronize()
    assert torch.equal(flat.scores[:, :flat.n_cols], paged.scores[:, :paged.n_cols])
    pl.page_table[0, 10] = pl.n_pages + 2      # past the pool: missing
    paged.index_scores(0, pool=False)
    torch.cuda.synchronize()
    g = _np(paged.scores)
    assert np.all(g[:, 640:704] == -np.inf)
    assert np.array_equal(g[:, :640], _np(flat.scores)[:, :640])


# ---------------------------------------------------------------------------
# a decoder group over the paged layout

@pytest.mark.parametrize("concurrent,rescore", [(False, None), (True, None), (True, True)])
def test_paged_group_equals_flat(concurrent, rescore):
    """The paged group equals the flat one (default route, one stream), also
    overlapped (the Full layer's top-k and attention on the second stream)
    and on the re-scoring route (the best blocks' keys scored again through
    the page table, their top-k writing slots)."""
    _announce(f"group full/reuse/reindex/reuse, paged + slots + inverse RoPE, "
              f"concurrent={concurrent} rescore={rescore}")
    wl = synth.mini_workload(78, [6000, 3333], q_per_seq=2,
                             modes=("full", "reuse", "reindex", "reuse"),
                             topk=128, n_blocks=60).to(DEV)
    pl = synth.paged_layout(wl, 79)
    flat = LayerRunner(wl, rope_cs=pl.rope_cs)
    paged = LayerRunner(wl, paged=pl, rescore=rescore)
    assert paged.rescored(0) == bool(rescore) and not flat.rescored(0)
    flat.run()
    paged.run(concurrent=concurrent)
    torch.cuda.synchronize()
    table = _np(pl.page_table)
    q_seq = _np(wl.q_seq)
    for li in flat.idx:
        assert np.array_equal(_np(paged.idx[li]),
                              oracle.slots_from_positions(_np(flat.idx[li]), q_seq, table))
    for li in range(len(wl.layers)):
        assert torch.equal(paged.out[li], flat.out[li]), li
        assert torch.equal(paged.lse[li], flat.lse[li]), li


def test_attention_slots_outside_the_pool_are_skipped():
    _announce("attention by slot, entries outside the pool")
    wl = synth.mini_workload(80, [1000], q_per_seq=2).to(DEV)
    pl = synth.paged_layout(wl, 81)
    paged = LayerRunner(wl, paged=pl, rope_cs=None)
    paged.rope_cs = None
    flat = LayerRunner(wl)
    idx = np.full((2, 512), -1, dtype=np.int64)
    idx[:, :100] = np.arange(100)
    slots = oracle.slots_from_positions(idx, _np(wl.q_seq), _np(pl.page_table))
    slots_bad = slots.copy()
    slots_bad[:, 100:110] = paged.n_main_rows + np.arange(10)   # past the pool
    flat.slots.topk_idxs = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    paged.slots.topk_idxs = torch.from_numpy(slots_bad.astype(np.int32)).to(DEV)
    flat.attention(0)
    paged.attention(0)
    torch.cuda.synchronize()
    assert torch.equal(flat.out[0], paged.out[0])
