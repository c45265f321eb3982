"""Parity at the five configurations' full sizes, in the launch configuration
the benchmark times.  Every stage runs on the whole workload; the oracle then
checks sampled queries stage by stage, each fed the GPU's own upstream
outputs (scores for selection, the pool for pool scoring, the indices for
attention), plus the end-to-end top-k sets against the oracle's own float64
scores with the gap rule."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_long_amd as tsl
from top_sparse_long_amd.driver import LayerRunner
from tests import oracle_io
from tests.parity import check_scores, check_index_table, check_topk_gap, check_attention, row_tau

pytestmark = pytest.mark.gpu
DEV = "cuda"

# Sampled queries: every query of the decode batches and of the 64-query
# group; on the 4,096-query chunk, every 64th query plus both sides of the
# boundaries where a kernel's query tiling or its workgroup-to-XCD mapping
# changes (the scorer's 16-query tiles; the attention's workgroups, dealt to
# the 8 XCDs in runs of 512), plus the ends.
SAMPLES = {"tiny_full_fp32": None, "decode_128k": list(range(8)),
           "prefill_m2_chunk": sorted(set(range(0, 4096, 64)) | {1, 15, 16, 17, 511, 512, 1023, 1024, 2047,
                                                                 2048, 3071, 3072, 4094, 4095}),
           "reindex_1m": [0, 1], "decoder_group_256k": list(range(64)),
           "decode_128k_pages_formats": list(range(8))}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsl.load()


def _np(t):
    return t.detach().cpu().numpy()


def _seq_keys(wl, b, n):
    base = int(wl.seq_base[b])
    rows = torch.arange(base, base + n, device=wl.k_idx.device)
    return oracle_io.index_k_rows(wl, rows)


def _gathered_main(wl, b, idx_row, n_vis):
    """Decode only the main rows a query's indices name; return them with
    the indices renumbered into that compact array."""
    sel = idx_row[idx_row >= 0]
    assert np.all(sel < n_vis), "an index beyond the visible prefix"
    rows = torch.from_numpy(int(wl.seq_base[b]) + sel).to(wl.main_kv.device)
    compact = np.full_like(idx_row, -1)
    compact[:len(sel)] = np.arange(len(sel))
    return oracle_io.main_rows(wl, rows), compact


def _check_rescore_route(run, wl, t, ref, idx_row, pos1, n):
    """Query t of a Full layer that wrote only block maxima: the maxima meet
    the score bound against the oracle's; the best blocks are the k best of
    the GPU's maxima (exact); their re-scored keys meet the score bound; the
    top-k is the exact top-k of those keys and, against the oracle's float64
    scores, meets the gap rule; the pool is the candidate ranking of the
    GPU's maxima (exact)."""
    bs = wl.block_size
    nb = -(-n // bs)
    bm = _np(run.block_max[t, :nb]).astype(np.float64)
    ref_bm = oracle.block_maxima(ref[0], n, bs)
    tau = row_tau(ref[0])
    fin = np.isfinite(ref_bm)
    assert np.array_equal(np.isfinite(bm), fin)
    assert np.all(np.abs(bm[fin] - ref_bm[fin]) <= 1e-3 * (np.abs(ref_bm[fin]) + tau))
    order = sorted(range(nb), key=lambda b: (-bm[b], b))
    want = sorted(b for b in order[:wl.topk] if bm[b] > -np.inf)
    tb = _np(run.top_blocks[t])
    assert [int(x) for x in tb if x >= 0] == want
    ts = _np(run.top_scores[t:t + 1, :run.top_cols])
    pos = oracle.pool_positions(tb[None], bs)[0]
    ref_ts = np.where((pos >= 0) & (pos < n), ref[0][np.clip(pos, 0, ref.shape[1] - 1)], -np.inf)
    check_scores(ts, ref_ts[None], "re-scored keys")
    assert np.array_equal(idx_row, oracle.topk_rows_pool(ts.astype(np.float64), tb[None], bs, wl.topk)[0])
    check_topk_gap(idx_row, ref[0, :n], np.arange(n), wl.topk, tau)
    # the pool: a score row whose blocks hold the GPU maxima (first column)
    row = np.full(ref.shape[1], -np.inf)
    row[np.arange(nb) * bs] = bm
    assert np.array_equal(_np(run.cand[t:t + 1]), oracle.block_candidates(row[None], pos1, wl.ratio, bs,
                                                                          wl.n_blocks))


# Every workload on the route the benchmark times (overlap_route: a
# pool-building Full layer of a decode batch re-scores its best blocks), and
# the 128K decode step also on the single-stream default route (dense scores,
# top-k and pool in shared launches).
CONFIG_CASES = ([(n, True) for n in list(synth.CONFIG_NAMES) + list(synth.EXTRA_WORKLOADS)]
                + [("decode_128k", False)])


@pytest.mark.parametrize("name,overlap_route", CONFIG_CASES)
def test_config_parity(name, overlap_route):
    print(f"[case] config {name} overlap_route={overlap_route}", flush=True)
    gen_dev = "cpu" if name == "tiny_full_fp32" else DEV
    wl = synth.make_workload(name, device=gen_dev).to(DEV)
    run = LayerRunner(wl)
    sample = SAMPLES[name] if SAMPLES[name] is not None else list(range(wl.Q))
    q_seq, q_pos = _np(wl.q_seq), _np(wl.q_pos)
    nvis = oracle.visible_count(q_pos, wl.ratio)
    quant = wl.quantized
    # per-sequence dequantized caches for the sampled queries only
    keys = {}
    for t in sample:
        b = int(q_seq[t])
        if b not in keys:
            keys[b] = _seq_keys(wl, b, int(wl.n_entries[b]))
    zero = np.zeros(1, dtype=np.int64)

    def sub(t):
        return keys[int(q_seq[t])], np.array([q_pos[t]]), np.array([0])

    # the benchmark's own call sequence, checked after each layer's attention
    steps = iter(run.steps(overlap_route=overlap_route))
    for li, lay in enumerate(wl.layers):
        print(f"[case] config {name} layer {li} ({lay.mode})", flush=True)
        for step_name, fn in steps:
            fn()
            if step_name == "sparse_attn":
                break
        torch.cuda.synchronize()
        idx = _np(run.slots.topk_idxs)[sample]
        check_index_table(idx, wl.topk)
        if lay.mode in ("full", "reindex"):
            qi = oracle_io.index_q(lay, quant)[sample]
            wi = oracle_io.index_w(lay, quant)[sample]
        sel = torch.tensor(sample, device=lay.q.device)
        qa = (oracle.decode_bf16(_np(lay.q[sel])) if quant
              else _np(lay.q[sel]).astype(np.float64))
        swa = oracle_io.swa_rows(lay, quant)
        for j, t in enumerate(sample):
            kr, pos1, seq0 = sub(t)
            n = int(nvis[t])
            if run.rescored(li, overlap_route):
                # the re-scoring route: block maxima only, the best blocks'
                # keys scored again
                ref = oracle.index_scores_dense(qi[j:j + 1], wi[j:j + 1], kr, zero, seq0, pos1,
                                                wl.ratio, run.n_cols)
                _check_rescore_route(run, wl, t, ref, idx[j], pos1, n)
            elif lay.mode == "full":
                ref = oracle.index_scores_dense(qi[j:j + 1], wi[j:j + 1], kr, zero, seq0, pos1,
                                                wl.ratio, run.n_cols)
                g = _np(run.scores[t:t + 1, :run.n_cols])
                check_scores(g, ref)
                g64 = g.astype(np.float64)
                assert np.array_equal(idx[j], oracle.topk_rows_dense(g64, pos1, wl.ratio, wl.topk)[0])
                check_topk_gap(idx[j], ref[0, :n], np.arange(n), wl.topk, row_tau(ref[0]))
                if run.needs_pool[li]:
                    cand = _np(run.cand[t:t + 1])
                    assert np.array_equal(cand, oracle.block_candidates(g64, pos1, wl.ratio, 8,
                                                                        wl.n_blocks))
            elif lay.mode == "reindex":
                cand = _np(run.cand[t:t + 1])
                ref = oracle.index_scores_pool(qi[j:j + 1], wi[j:j + 1], kr, zero, seq0, pos1,
                                               wl.ratio, cand, 8)
                g = _np(run.pool_scores[t:t + 1, :run.pool_cols])
                check_scores(g, ref, "pool scores")
                assert np.array_equal(idx[j], oracle.topk_rows_pool(g.astype(np.float64), cand, 8,
                                                                    wl.topk)[0])
                members = oracle.pool_positions(cand, 8)[0]
                ok = members >= 0
                check_topk_gap(idx[j], np.where(ok, ref[0], -np.inf), np.where(ok, members, 0),
                               wl.topk, row_tau(ref[0]))
            # attention on the GPU's indices
            b = int(q_seq[t])
            mr, cidx = _gathered_main(wl, b, idx[j], n)
            out, lse = oracle.sparse_attn(qa[j:j + 1], mr, zero,
                                          cidx[None], swa, _np(wl.swa_base)[b:b + 1],
                                          _np(wl.swa_pos0)[b:b + 1], None, wl.window, seq0, pos1,
                                          _np(lay.sink).astype(np.float64), wl.softmax_scale,
                                          wl.ratio)
            check_attention(_np(run.out[li][t:t + 1].float()), out, f"{name} layer {li} query {t}")
            assert np.abs(_np(run.lse[li][t]) - lse[0]).max() < 1e-3
        if name == "tiny_full_fp32" and lay.mode == "full":
            # integer inputs: fp32 scores are exact, so the whole pipeline is exact
            assert np.array_equal(_np(run.scores[:, :run.n_cols]).astype(np.float64),
                                  oracle.index_scores_dense(oracle_io.index_q(lay, False),
                                                            oracle_io.index_w(lay, False),
                                                            oracle_io.index_k_rows(wl),
                                                            _np(wl.seq_base), q_seq, q_pos, 1,
                                                            run.n_cols))


@pytest.mark.parametrize("name", [n for n in list(synth.CONFIG_NAMES) + list(synth.EXTRA_WORKLOADS)
                                  if n != "tiny_full_fp32"])
def test_config_serving_io_equals_flat(name):
    """Full size, serving-shaped I/O (DSA page, top-k section): the caches in
    64-slot pages of random order, the top-k writing slots, attention by slot
    with the inverse RoPE.  Against the flat run with the same RoPE table:
    every top-k table is the oracle's translation of the flat positions and
    every layer's output and LSE are bit-identical."""
    print(f"[case] serving I/O at full size: {name}", flush=True)
    wl = synth.make_workload(name, device=DEV)
    pl = synth.paged_layout(wl, 11)
    flat = LayerRunner(wl, rope_cs=pl.rope_cs)
    paged = LayerRunner(wl, paged=pl)
    flat.run()
    paged.run()
    torch.cuda.synchronize()
    table = _np(pl.page_table)
    q_seq = _np(wl.q_seq)
    for li in flat.idx:
        fidx = _np(flat.idx[li])
        want = oracle.slots_from_positions(fidx, q_seq, table)
        assert (fidx >= 0).sum() > 0 and np.any(want != fidx), li   # real selections, translated
        assert np.array_equal(_np(paged.idx[li]), want), li
    for li in range(len(wl.layers)):
        assert torch.equal(paged.out[li], flat.out[li]), li
        assert torch.equal(paged.lse[li], flat.lse[li]), li
