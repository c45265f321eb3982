"""Pins of the oracle's compressor, layer-role arithmetic and slot driver."""
import json
import os

import numpy as np
import torch

import oracle
import synth
from tests import oracle_io

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_compressor_ratio_one_is_identity():
    """xhh.club three-modes page: with m = 1 the softmax weight is identically
    1 and there is no Z projection."""
    c = np.random.default_rng(0).normal(size=(7, 5))
    assert np.array_equal(oracle.compress(c, None, 1), c)


def test_compressor_ratio_two_weights():
    """m = 2: weights are sigmoid(+-(z0 - z1)) per channel and sum to one."""
    rng = np.random.default_rng(1)
    z = rng.normal(size=(6, 4))
    ones = oracle.compress(np.ones((6, 4)), z, 2)
    assert np.allclose(ones, 1.0)
    c = rng.normal(size=(6, 4))
    got = oracle.compress(c, z, 2)
    sig = 1.0 / (1.0 + np.exp(-(z[0::2] - z[1::2])))
    assert np.allclose(got, sig * c[0::2] + (1 - sig) * c[1::2], rtol=1e-13)
    # an odd trailing token has no entry yet
    assert oracle.compress(c[:5], z[:5], 2).shape == (2, 4)


def test_generator_compressor_agrees_with_oracle():
    g = torch.Generator().manual_seed(3)
    c = torch.randn(64, 512, generator=g)
    z = torch.randn(64, 512, generator=g)
    got = synth.workloads.compress_pairs_input(c, z).double().numpy()
    ref = oracle.compress(c.double().numpy(), z.double().numpy(), 2)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)


def test_pages_arithmetic():
    g = json.load(open(os.path.join(GOLD, "pages_arithmetic.json")))
    e = g["global_entries_per_token"]
    assert oracle.global_entries_per_token(e["full_layer_ratios"]) == e["value"]
    p = g["pool_positions"]
    full = np.arange(p["blocks"])[None]
    assert oracle.pool_positions(full, p["block_size"]).shape[1] == p["value"]
    cov = g["pool_coverage_1m"]
    assert round(100.0 * p["value"] / cov["context"], 1) == cov["value_percent"]
    assert cov["context"] // p["block_size"] == 125000
    h = g["fp4_headroom"]
    finite = oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)]
    assert finite.max() * oracle.E2M1_TABLE.max() == h["value"]
    ik = g["index_k_bytes"]
    assert 128 * 1 + 4 == ik["value"] and ik["page_slots"] * ik["value"] == ik["page_bytes"]
    assert synth.SWA_RECORD_BYTES == g["swa_record_bytes"]["value"]
    oracle.decode_swa_records(np.zeros((1, g["swa_record_bytes"]["value"]), np.uint8))


def test_slot_driver_semantics():
    """xhh.club three-modes page, 'shared pool mechanism': Full writes the
    slots, Reindex rewrites topk_idxs from the pool, Reuse only reads."""
    wl = synth.mini_workload(5, [3000, 2500], q_per_seq=2, quantized=True,
                             modes=("full", "reuse", "reindex", "reuse"),
                             topk=64, n_blocks=40)
    res = oracle_io.run_oracle(wl)
    assert np.array_equal(res[0]["idx"], res[1]["idx"])
    assert np.array_equal(res[2]["idx"], res[3]["idx"])
    assert not np.array_equal(res[0]["idx"], res[2]["idx"])
    members = oracle.pool_positions(res[0]["candidates"], 8)
    for t in range(wl.Q):
        sel = res[2]["idx"][t]
        assert set(sel[sel >= 0]) <= set(members[t][members[t] >= 0])
    # layers own their q, SWA and sink: Reuse outputs differ from Full's
    assert not np.allclose(res[0]["out"], res[1]["out"])


def test_slot_driver_short_sequences_pool_equals_dense():
    wl = synth.mini_workload(6, [700, 333], q_per_seq=1, quantized=True,
                             modes=("full", "reindex"))
    a = oracle_io.run_oracle(wl, use_pool=True)
    b = oracle_io.run_oracle(wl, use_pool=False)
    assert np.array_equal(a[1]["idx"], b[1]["idx"])
    assert np.allclose(a[1]["out"], b[1]["out"], rtol=1e-13)
