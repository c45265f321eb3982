"""The allocation-free selection entry point against the workspace one.

csa2_topk_and_block_candidates_noalloc keeps its selection lists in the
library's static device buffer instead of a caller workspace.  Two calls in a
row, the second on a smaller input (so the buffer holds the first call's
lists when the second starts), must each equal
csa2_topk_and_block_candidates on the same scores bit for bit."""
import numpy as np
import pytest
import torch

import top_sparse_long_amd as tsl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsl.load()


def _case(seed, Q, n_cols, fuse):
    """Scores with many ties (integers), ragged rows, optional fused maxima."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    stride = (n_cols + 63) // 64 * 64
    scores = torch.randint(-300, 300, (Q, stride), generator=g, device=DEV).to(torch.float32)
    rng = np.random.default_rng(seed)
    q_pos = rng.integers(n_cols // 3, n_cols, size=Q)
    q_pos[0] = n_cols - 1
    q_pos = torch.from_numpy(q_pos.astype(np.int32)).to(DEV)
    bm = None
    if fuse:
        nb = (n_cols + 7) // 8
        bstride = (nb + 63) // 64 * 64
        vis = torch.arange(stride, device=DEV)[None, :] < (q_pos.to(torch.int64) + 1)[:, None]
        masked = torch.where(vis, scores, torch.full_like(scores, -float("inf")))
        bm = torch.full((Q, bstride), -float("inf"), device=DEV)
        bm[:, :nb] = masked[:, :nb * 8].reshape(Q, nb, 8).amax(-1)
    return scores, q_pos, bm


def _both(scores, q_pos, bm, n_cols, k=512, n_blocks=2048):
    Q = scores.shape[0]
    need = tsl.csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, 8, n_blocks)
    assert 0 < need <= tsl.csa2_noalloc_scratch_bytes()
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    idx_w = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    cand_w = torch.full((Q, n_blocks), -7, dtype=torch.int32, device=DEV)
    tsl.csa2_topk_and_block_candidates(scores, n_cols, q_pos, 1, k, idx_w, 8, n_blocks, cand_w, ws,
                                       Q, block_max=bm)
    idx_n = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
    cand_n = torch.full((Q, n_blocks), -9, dtype=torch.int32, device=DEV)
    tsl.csa2_topk_and_block_candidates_noalloc(scores, n_cols, q_pos, 1, k, idx_n, 8, n_blocks,
                                               cand_n, Q, block_max=bm)
    torch.cuda.synchronize()
    return idx_w, cand_w, idx_n, cand_n


@pytest.mark.parametrize("fuse", [False, True])
def test_noalloc_equals_workspace_call_twice_then_smaller(fuse):
    print(f"[case] noalloc selection fuse={fuse}", flush=True)
    # first: 8 rows of 131,072 columns (multi-stage top-k lists);
    # second: 3 rows of 50,000 (smaller lists over the first call's leftovers)
    for seed, Q, n_cols in ((1, 8, 131072), (2, 3, 50000)):
        scores, q_pos, bm = _case(seed, Q, n_cols, fuse)
        idx_w, cand_w, idx_n, cand_n = _both(scores, q_pos, bm, n_cols)
        assert torch.equal(idx_w, idx_n), (seed, Q, n_cols)
        assert torch.equal(cand_w, cand_n), (seed, Q, n_cols)
        # the rows are full (at least k visible), so no -1 in the top-k
        assert int((idx_n < 0).sum()) == 0
