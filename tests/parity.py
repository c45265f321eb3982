"""Comparison rules between the HIP path and the oracle.

* Index scores: |gpu - ref| <= 1e-3 * (|ref| + tau) with tau = 1e-2 * RMS of
  the row's finite reference scores (the floor keeps near-zero cancellations
  from dividing by ~0); the -inf pattern must match exactly.
* Index sets (top-k, pool): bit-exact where the oracle is fed the GPU's own
  fp32 scores; against the oracle's float64 scores, every element of the
  symmetric difference must score within delta = 1e-3 * (|T| + tau) of the
  oracle's k-th score T (identical sets whenever the k-th/k+1-th gap exceeds
  the score bound).
* Attention: max |gpu - ref| <= 1e-2 and ||gpu - ref|| / ||ref|| <= 5e-3 per
  query, against the float64 oracle run on the GPU's own indices.
"""
import numpy as np

import oracle

SCORE_REL = 1e-3
ATTN_MAX_ABS = 1e-2
ATTN_REL_L2 = 5e-3


def row_tau(ref_row):
    fin = ref_row[np.isfinite(ref_row)]
    return 1e-2 * float(np.sqrt(np.mean(fin ** 2))) if fin.size else 0.0


def check_scores(gpu, ref, what="scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    for t in range(ref.shape[0]):
        fin = np.isfinite(ref[t])
        assert np.array_equal(np.isfinite(gpu[t]), fin), f"{what}: -inf pattern differs in row {t}"
        assert np.all(gpu[t][~fin] == -np.inf), f"{what}: non -inf masked entries in row {t}"
        if not fin.any():
            continue
        tau = row_tau(ref[t])
        err = np.abs(gpu[t][fin] - ref[t][fin]) / (SCORE_REL * (np.abs(ref[t][fin]) + tau))
        worst = float(err.max())
        assert worst <= 1.0, f"{what}: row {t} relative error {worst * SCORE_REL:.3g} over the bound"


def check_index_table(idx, k):
    """Ascending valid entries, then -1 padding."""
    idx = np.asarray(idx)
    for row in idx:
        n = int((row >= 0).sum())
        assert np.all(row[:n] >= 0) and np.all(row[n:] == -1), "padding not at the end"
        assert np.all(np.diff(row[:n]) > 0), "entries not strictly ascending"


def check_topk_gap(gpu_row, values, positions, k, tau):
    """gpu_row: the GPU's top-k positions; values/positions: the oracle's
    float64 scores of the candidates and their positions."""
    ref = oracle.topk(values, positions, k)
    G = set(int(x) for x in gpu_row if x >= 0)
    O = set(int(x) for x in ref if x >= 0)
    assert len(G) == len(O), (len(G), len(O))
    if G == O:
        return 0
    vals = dict(zip((int(p) for p in positions), values))
    order = oracle._first_k_by_score(values, positions, k)
    T = float(values[order[-1]])
    delta = SCORE_REL * (abs(T) + tau)
    for x in G ^ O:
        assert abs(vals[x] - T) <= delta, f"position {x} score {vals[x]} vs k-th {T} (delta {delta})"
    return len(G ^ O)


def check_attention(gpu, ref, what="attention"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    for t in range(ref.shape[0]):
        d = gpu[t] - ref[t]
        mx = float(np.abs(d).max())
        rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref[t]), 1e-30))
        assert mx <= ATTN_MAX_ABS, f"{what}: query {t} max abs error {mx:.3g}"
        assert rel <= ATTN_REL_L2, f"{what}: query {t} relative L2 error {rel:.3g}"
