"""The C-ABI library loads, exports what include/csa2.h declares, and rejects
bad arguments on the host (no GPU needed: every call here fails its host
checks before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import top_sparse_long_amd as tsl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tsl.load()
    names = _declared()
    assert set(tsl.EXPORTED) == set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = tsl.load()
    assert lib.csa2_version() >= 100
    assert lib.csa2_status_string(0) == b"CSA2_OK"
    assert lib.csa2_status_string(-3) == b"CSA2_ERR_WORKSPACE"
    assert lib.csa2_status_string(7) == b"CSA2_ERR_UNKNOWN"


FAKE = 0x100000   # never dereferenced: every call below fails a host check


def _rows(dtype, stride=128, scale=True):
    return tsl.csa2_rows(FAKE, FAKE if scale else None, stride, 1, dtype)


def _scores(lib, **kw):
    a = dict(q=_rows(tsl.CSA2_FP8_E4M3), w=FAKE, wdt=tsl.CSA2_BF16, k=_rows(tsl.CSA2_FP8_E4M3),
             seq_base=FAKE, q_seq=FAKE, q_pos=FAKE, ratio=1, cand=None, ncb=0, bs=8,
             scores=FAKE, stride=1024, n_cols=1024, bmax=None, bms=0, Q=1, H=32, d=128,
             pages=None)
    a.update(kw)
    st = lib.csa2_index_scores(ctypes.byref(a["q"]), a["w"], a["wdt"], ctypes.byref(a["k"]),
                               a["seq_base"], a["q_seq"], a["q_pos"], a["ratio"], a["cand"],
                               a["ncb"], a["bs"], a["scores"], a["stride"], a["n_cols"],
                               a["bmax"], a["bms"], a["Q"], a["H"], a["d"],
                               None if a["pages"] is None else ctypes.byref(a["pages"]), None)
    return st, lib.csa2_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(scores=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(q_pos=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(Q=-1), tsl.CSA2_ERR_INVALID_ARG),
    (dict(ratio=3), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(d=64), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(H=64), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(wdt=tsl.CSA2_FP8_E4M3), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(k=_rows(tsl.CSA2_F32, 512, False)), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(stride=1000), tsl.CSA2_ERR_INVALID_ARG),
    (dict(stride=1022), tsl.CSA2_ERR_INVALID_ARG),
    (dict(scores=FAKE + 4), tsl.CSA2_ERR_INVALID_ARG),
    (dict(q=_rows(tsl.CSA2_FP8_E4M3, 130)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(cand=FAKE, ncb=100, bs=8), tsl.CSA2_ERR_INVALID_ARG),
    (dict(cand=FAKE, ncb=128, bs=6, n_cols=768), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(q=_rows(tsl.CSA2_FP8_E4M3, scale=False), k=_rows(tsl.CSA2_FP8_E4M3, scale=False)),
     tsl.CSA2_ERR_INVALID_ARG),
    (dict(bmax=FAKE, bms=64), tsl.CSA2_ERR_INVALID_ARG),
    (dict(bmax=FAKE, bms=128, bs=64), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(bmax=FAKE, bms=128, cand=FAKE, ncb=128), tsl.CSA2_ERR_INVALID_ARG),
])
def test_index_scores_rejects(kw, status):
    st, msg = _scores(tsl.load(), **kw)
    assert st == status and msg.startswith("csa2_index_scores")


def test_topk_rejects():
    lib = tsl.load()
    assert lib.csa2_topk(None, 64, 64, FAKE, 1, None, 0, 8, 8, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert lib.csa2_topk(FAKE, 64, 64, FAKE, 1, None, 0, 8, 4096, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert lib.csa2_topk(FAKE, 64, 64, FAKE, 1, None, 0, 8, 0, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert lib.csa2_topk(FAKE, 32, 64, FAKE, 1, None, 0, 8, 8, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert lib.csa2_topk(FAKE, 64, 64, FAKE, 5, None, 0, 8, 8, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    # long rows need a workspace
    need = lib.csa2_topk_workspace_size(4, 200000, 512)
    assert need > 0
    st = lib.csa2_topk(FAKE, 200000, 200000, FAKE, 1, None, 0, 8, 512, FAKE, FAKE, need - 1, 4, None, None)
    assert st == tsl.CSA2_ERR_WORKSPACE
    assert "workspace" in lib.csa2_last_error().decode()


def test_block_candidates_rejects():
    lib = tsl.load()
    bc = lib.csa2_block_candidates
    assert bc(FAKE, 64, 64, None, 0, None, 1, 8, 16, FAKE, None, 0, 1, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert bc(FAKE, 64, 64, None, 0, FAKE, 1, 12, 16, FAKE, None, 0, 1, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert bc(FAKE, 64, 64, None, 0, FAKE, 1, 8, 8192, FAKE, None, 0, 1, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert bc(FAKE + 4, 64, 64, None, 0, FAKE, 1, 8, 16, FAKE, None, 0, 1, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    # with block maxima the scores are not needed, but the maxima stride is checked
    assert bc(None, 0, 64, FAKE, 4, FAKE, 1, 8, 16, FAKE, None, 0, 1, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    need = lib.csa2_block_candidates_workspace_size(2, 1 << 20, 8, 2048)
    assert need > 0
    assert bc(FAKE, 1 << 20, 1 << 20, None, 0, FAKE, 1, 8, 2048, FAKE, FAKE, 0, 2, None) == \
        tsl.CSA2_ERR_WORKSPACE


def test_topk_and_block_candidates_rejects():
    lib = tsl.load()
    f = lib.csa2_topk_and_block_candidates
    # scores, q_pos, block size, k and the pool size are checked as in the separate calls
    assert f(None, 64, 64, None, 0, FAKE, 1, 8, FAKE, 8, 16, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 64, 64, None, 0, None, 1, 8, FAKE, 8, 16, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 64, 64, None, 0, FAKE, 1, 8, FAKE, 12, 16, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert f(FAKE, 64, 64, None, 0, FAKE, 1, 4096, FAKE, 8, 16, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert f(FAKE, 64, 64, None, 0, FAKE, 1, 8, FAKE, 8, 8192, FAKE, None, 0, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    # the workspace holds both selections' lists
    Q, n = 2, 1 << 20
    need = lib.csa2_topk_and_block_candidates_workspace_size(Q, n, 512, 8, 2048)
    t = lib.csa2_topk_workspace_size(Q, n, 512)
    b = lib.csa2_block_candidates_workspace_size(Q, n, 8, 2048)
    assert t > 0 and b > 0 and need >= t + b and need - (t + b) < 16
    for short in (need - 1, t, 0):
        assert f(FAKE, n, n, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, FAKE, short, Q, None, None) == \
            tsl.CSA2_ERR_WORKSPACE
    assert f(FAKE, n, n, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, FAKE + 4, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    # Q == 0 passes every check and enqueues nothing
    assert f(FAKE, n, n, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, None, 0, 0, None, None) == tsl.CSA2_OK


def test_topk_from_block_max_rejects():
    lib = tsl.load()
    f = lib.csa2_topk_from_block_max
    n, Q, k = 32768, 4, 512
    nb = n // 8
    need = lib.csa2_topk_from_block_max_workspace_size(Q, n, k, 8)
    assert need >= Q * k * 8
    # block maxima are required, 4-byte aligned, with a stride covering every block
    assert f(FAKE, n, n, None, 0, FAKE, 1, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, n, n, FAKE, nb - 1, FAKE, 1, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, n, n, FAKE + 2, nb, FAKE, 1, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    # q_pos is required; the block size is a power of two up to 32
    assert f(FAKE, n, n, FAKE, nb, None, 1, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    for bs in (12, 64):
        assert f(FAKE, n, n, FAKE, n, FAKE, 1, bs, k, FAKE, FAKE, need, Q, None, None) == \
            tsl.CSA2_ERR_UNSUPPORTED
    # the workspace holds the k best blocks of every row
    assert f(FAKE, n, n, FAKE, nb, FAKE, 1, 8, k, FAKE, FAKE, need - 1, Q, None, None) == \
        tsl.CSA2_ERR_WORKSPACE
    assert f(FAKE, n, n, FAKE, nb, FAKE, 1, 8, k, FAKE, FAKE + 4, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    # the plain top-k's checks apply (k, ratio, scores)
    assert f(FAKE, n, n, FAKE, nb, FAKE, 1, 8, 4096, FAKE, FAKE, 1 << 30, Q, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert f(FAKE, n, n, FAKE, nb, FAKE, 3, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    assert f(None, n, n, FAKE, nb, FAKE, 1, 8, k, FAKE, FAKE, need, Q, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    # k * block_size above 32,768 takes the dense top-k and its workspace size
    big = 300000
    assert lib.csa2_topk_from_block_max_workspace_size(Q, big, 2048, 32) == \
        lib.csa2_topk_workspace_size(Q, big, 2048)
    # the block ranking's lists, else the k best blocks of every row
    assert lib.csa2_topk_from_block_max_workspace_size(Q, big, 2048, 8) == \
        max(lib.csa2_topk_workspace_size(Q, -(-big // 8), 2048), Q * 2048 * 8)
    assert lib.csa2_topk_from_block_max_workspace_size(Q, 4096, 512, 8) == Q * 512 * 8
    # Q == 0 passes every check and enqueues nothing
    assert f(FAKE, n, n, FAKE, nb, FAKE, 1, 8, k, FAKE, None, 0, 0, None, None) == tsl.CSA2_OK


def test_diag_stream_read_and_write_reject():
    lib = tsl.load()
    f = lib.csa2_diag_stream_read
    assert f(None, 1024, FAKE, 16, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 1024, None, 16, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE + 4, 1024, FAKE, 16, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 1000, FAKE, 16, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 1024, FAKE, 0, None) == tsl.CSA2_ERR_INVALID_ARG
    # nothing to read: nothing is enqueued
    assert f(FAKE, 0, FAKE, 16, None) == tsl.CSA2_OK
    w = lib.csa2_diag_stream_write
    assert w(None, 1024, 0.0, None) == tsl.CSA2_ERR_INVALID_ARG
    assert w(FAKE + 8, 1024, 0.0, None) == tsl.CSA2_ERR_INVALID_ARG
    assert w(FAKE, 1000, 0.0, None) == tsl.CSA2_ERR_INVALID_ARG
    assert w(FAKE, 0, 0.0, None) == tsl.CSA2_OK


def test_top_blocks_and_block_candidates_rejects():
    lib = tsl.load()
    f = lib.csa2_top_blocks_and_block_candidates
    n = 1 << 23   # 1M blocks of 8: ranked in stages, through the workspace
    ws = lib.csa2_top_blocks_and_block_candidates_workspace_size(2, n, 8, 64, 128)
    assert ws > 0
    ok = (FAKE, n // 8, n, FAKE, 1, 8, 64, FAKE, 128, FAKE, FAKE, ws, 2, None)
    for i in (0, 3, 7, 9):   # block_max, q_pos, top_blocks, cand
        args = list(ok)
        args[i] = None
        assert f(*args) == tsl.CSA2_ERR_INVALID_ARG, i
    bad = list(ok)
    bad[5] = 6   # block_size not a power of two
    bad[1] = n
    assert f(*bad) == tsl.CSA2_ERR_UNSUPPORTED
    bad = list(ok)
    bad[6] = 5000   # k_blocks above 4096
    assert f(*bad) == tsl.CSA2_ERR_UNSUPPORTED
    bad = list(ok)
    bad[1] = n // 8 - 1   # block_max stride below the block count
    assert f(*bad) == tsl.CSA2_ERR_INVALID_ARG
    bad = list(ok)
    bad[11] = ws - 16   # short workspace
    assert f(*bad) == tsl.CSA2_ERR_WORKSPACE
    # nothing to rank: nothing is enqueued
    zero = list(ok)
    zero[12] = 0
    assert f(*zero) == tsl.CSA2_OK


def test_diag_mfma_valu_rejects():
    lib = tsl.load()
    f = lib.csa2_diag_mfma_valu
    n = 256 * 512
    assert f(1, 10, None, n, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(0, 10, FAKE, n, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(4, 10, FAKE, n, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(3, 0, FAKE, n, None) == tsl.CSA2_ERR_INVALID_ARG
    assert f(3, 10, FAKE, n - 1, None) == tsl.CSA2_ERR_INVALID_ARG


def test_topk_and_block_candidates_noalloc_rejects_sizes_past_the_scratch():
    """The allocation-free variant refuses, before anything is enqueued, any
    shape whose selection lists exceed its static buffer; its other argument
    checks are those of the workspace call."""
    lib = tsl.load()
    f = lib.csa2_topk_and_block_candidates_noalloc
    cap = lib.csa2_noalloc_scratch_bytes()
    assert cap == 16 << 20
    Q, n = 64, 1 << 20
    need = lib.csa2_topk_and_block_candidates_workspace_size(Q, n, 512, 8, 2048)
    assert need > cap
    assert f(FAKE, n, n, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, Q, None, None) == \
        tsl.CSA2_ERR_WORKSPACE
    assert b"static buffer" in lib.csa2_last_error()
    # shapes that fit still meet the ordinary checks first (null scores, bad block size)
    assert lib.csa2_topk_and_block_candidates_workspace_size(8, 1 << 17, 512, 8, 2048) <= cap
    assert f(None, 1 << 17, 1 << 17, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, 8, None, None) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert f(FAKE, 64, 64, None, 0, FAKE, 1, 8, FAKE, 12, 16, FAKE, 1, None, None) == \
        tsl.CSA2_ERR_UNSUPPORTED
    # Q == 0 needs no scratch and enqueues nothing
    assert f(FAKE, n, n, None, 0, FAKE, 1, 512, FAKE, 8, 2048, FAKE, 0, None, None) == tsl.CSA2_OK


def test_index_scores_fp4_key_checks():
    """FP4 keys with E4M3 scales: only beside FP8 queries, scales 4-byte aligned
    with a stride of at least 8 bytes."""
    lib = tsl.load()
    q = tsl.csa2_rows(FAKE, FAKE, 128, 1, tsl.CSA2_FP8_E4M3)
    k_ok = tsl.csa2_rows(FAKE, FAKE, 64, 8, tsl.CSA2_FP4_E2M1_E4M3S16)

    def call(qr, kr, Q=1):
        return lib.csa2_index_scores(ctypes.byref(qr), FAKE, tsl.CSA2_BF16, ctypes.byref(kr), FAKE,
                                     FAKE, FAKE, 1, None, 0, 8, FAKE, 64, 64, None, 0, Q, 32, 128,
                                     None, None)
    assert call(q, k_ok, Q=0) == tsl.CSA2_OK
    assert call(q, tsl.csa2_rows(FAKE, FAKE + 2, 64, 8, tsl.CSA2_FP4_E2M1_E4M3S16)) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert call(q, tsl.csa2_rows(FAKE, FAKE, 64, 4, tsl.CSA2_FP4_E2M1_E4M3S16)) == \
        tsl.CSA2_ERR_INVALID_ARG
    assert call(q, tsl.csa2_rows(FAKE, FAKE, 48, 8, tsl.CSA2_FP4_E2M1_E4M3S16)) == \
        tsl.CSA2_ERR_INVALID_ARG
    qf = tsl.csa2_rows(FAKE, None, 512, 0, tsl.CSA2_F32)
    assert call(qf, k_ok) == tsl.CSA2_ERR_UNSUPPORTED


def test_workspace_sizes():
    lib = tsl.load()
    assert lib.csa2_topk_workspace_size(64, 32768, 512) == 0      # one chunk per row
    assert lib.csa2_topk_workspace_size(8, 131072, 512) > 0
    assert lib.csa2_block_candidates_workspace_size(64, 262144, 8, 2048) == 0
    assert lib.csa2_block_candidates_workspace_size(2, 1 << 20, 8, 2048) > 0
    assert lib.csa2_topk_workspace_size(0, 100, 5) == 0


def _attn(lib, **kw):
    a = dict(q=FAKE, qdt=tsl.CSA2_BF16, main=tsl.csa2_rows(FAKE, FAKE, 320, 80, tsl.CSA2_FP4_E2M1),
             main_base=FAKE, idx=FAKE, k=512,
             swa=tsl.csa2_rows(FAKE, FAKE + 512, 528, 132, tsl.CSA2_FP8_E4M3),
             swa_base=FAKE, swa_pos0=FAKE, swa_lo=None, window=128, q_seq=FAKE, q_pos=FAKE,
             ratio=1, sink=FAKE, scale=0.044, out=FAKE, odt=tsl.CSA2_BF16, lse=None, ws=None,
             wsb=0, Q=1, H=64, D=512, io=None)
    a.update(kw)
    return lib.csa2_sparse_attn(a["q"], a["qdt"], ctypes.byref(a["main"]), a["main_base"],
                                a["idx"], a["k"], ctypes.byref(a["swa"]), a["swa_base"],
                                a["swa_pos0"], a["swa_lo"], a["window"], a["q_seq"], a["q_pos"],
                                a["ratio"], a["sink"], ctypes.c_float(a["scale"]), a["out"],
                                a["odt"], a["lse"], a["ws"], a["wsb"], a["Q"], a["H"], a["D"],
                                None if a["io"] is None else ctypes.byref(a["io"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(sink=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(D=576), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(H=40), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(k=4096), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(window=-1), tsl.CSA2_ERR_INVALID_ARG),
    (dict(qdt=tsl.CSA2_F32), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(odt=tsl.CSA2_FP8_E4M3), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(out=FAKE + 8), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, FAKE + 4, 320, 80, tsl.CSA2_FP4_E2M1)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, None, 320, 80, tsl.CSA2_FP4_E2M1)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(ratio=4), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(main=tsl.csa2_rows(FAKE, FAKE + 4, 288, 288, tsl.CSA2_FP4_E2M1_E4M3S16)),
     tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, FAKE + 256, 288, 20, tsl.CSA2_FP4_E2M1_E4M3S16)),
     tsl.CSA2_ERR_INVALID_ARG),
    (dict(ws=FAKE + 4, wsb=1 << 30), tsl.CSA2_ERR_INVALID_ARG),
    (dict(io=tsl.csa2_attn_io(FAKE + 4, 64, 0, 0)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(io=tsl.csa2_attn_io(FAKE, -1, 0, 0)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(io=tsl.csa2_attn_io(None, 0, 1, -5)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main_base=None), tsl.CSA2_ERR_INVALID_ARG),         # needed unless idx holds slots
])
def test_sparse_attn_rejects(kw, status):
    lib = tsl.load()
    assert _attn(lib, **kw) == status
    assert lib.csa2_last_error().decode().startswith("csa2_sparse_attn")


def test_attention_workspace_sizes():
    lib = tsl.load()
    one = 16 + 16 + 16 * 512
    # two queries of 64 heads: 8 groups of 16 heads x 4 column parts = 32
    # workgroups, so the 5 rounds of 128 keys are split four ways
    assert lib.csa2_sparse_attn_workspace_size(2, 64, 512, 128) == 2 * 4 * 4 * one * 4
    # from 128 workgroups (8 queries of 64 heads) on, nothing is split
    assert lib.csa2_sparse_attn_workspace_size(8, 64, 512, 128) == 0
    assert lib.csa2_sparse_attn_workspace_size(64, 64, 512, 128) == 0
    assert lib.csa2_sparse_attn_workspace_size(0, 64, 512, 128) == 0
    # a tiny key set needs no split either
    assert lib.csa2_sparse_attn_workspace_size(1, 16, 16, 0) == 0


def test_zero_queries_is_a_no_op_after_checks():
    lib = tsl.load()
    # Q == 0 passes every check and enqueues nothing, so it is safe without a GPU
    st, _ = _scores(lib, Q=0)
    assert st == tsl.CSA2_OK
    assert _attn(lib, Q=0) == tsl.CSA2_OK
    # slot indices need no main_base; an inverse-RoPE table passes the checks
    assert _attn(lib, Q=0, main_base=None, io=tsl.csa2_attn_io(None, 0, 1, 1 << 20)) == tsl.CSA2_OK
    assert _attn(lib, Q=0, io=tsl.csa2_attn_io(FAKE, 4096, 0, 0)) == tsl.CSA2_OK
    # the pages' 288-byte main-KV record passes the same checks
    assert _attn(lib, Q=0, main=tsl.csa2_rows(FAKE, FAKE + 256, 288, 288,
                                              tsl.CSA2_FP4_E2M1_E4M3S16)) == tsl.CSA2_OK


def _cw(lib, **kw):
    a = dict(c=FAKE, z=FAKE, stride=1024, seq=FAKE, pos=FAKE, T=4, ratio=2, pend=FAKE, B=2,
             kvw=FAKE, wik=FAKE, kw=FAKE, eps=1e-6, rope=FAKE, n_rope=64,
             main=tsl.csa2_rows(FAKE, FAKE + 256, 320, 80, tsl.CSA2_FP4_E2M1), mbase=FAKE,
             mrows=16, k=tsl.csa2_rows(FAKE, FAKE, 128, 1, tsl.CSA2_FP8_E4M3), kbase=FAKE,
             krows=16)
    a.update(kw)
    st = lib.csa2_cache_write(a["c"], a["z"], a["stride"], a["seq"], a["pos"], a["T"], a["ratio"],
                              a["pend"], a["B"], a["kvw"], a["wik"], a["kw"],
                              ctypes.c_float(a["eps"]), a["rope"], a["n_rope"],
                              None if a["main"] is None else ctypes.byref(a["main"]), a["mbase"],
                              a["mrows"], None if a["k"] is None else ctypes.byref(a["k"]),
                              a["kbase"], a["krows"], None)
    return st, lib.csa2_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(c=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(z=None), tsl.CSA2_ERR_INVALID_ARG),                 # ratio 2 needs the gates
    (dict(ratio=4), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(T=-1), tsl.CSA2_ERR_INVALID_ARG),
    (dict(seq=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(stride=1008), tsl.CSA2_ERR_INVALID_ARG),            # below one 512-value bf16 row
    (dict(stride=1032), tsl.CSA2_ERR_INVALID_ARG),            # not 16-byte aligned
    (dict(c=FAKE + 8), tsl.CSA2_ERR_INVALID_ARG),
    (dict(pend=FAKE + 4), tsl.CSA2_ERR_INVALID_ARG),
    (dict(eps=-1.0), tsl.CSA2_ERR_INVALID_ARG),
    (dict(eps=float("inf")), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=None, k=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(mbase=None), tsl.CSA2_ERR_INVALID_ARG),
    (dict(wik=None), tsl.CSA2_ERR_INVALID_ARG),               # index keys need W_IK
    (dict(kw=FAKE + 4), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, None, 320, 80, tsl.CSA2_FP4_E2M1)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, FAKE, 320, 8, tsl.CSA2_FP4_E2M1)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, FAKE, 288, 16, tsl.CSA2_FP4_E2M1_E4M3S16)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, None, 1024, 0, tsl.CSA2_F32)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(main=tsl.csa2_rows(FAKE, FAKE, 528, 132, tsl.CSA2_FP8_E4M3)), tsl.CSA2_ERR_UNSUPPORTED),
    (dict(k=tsl.csa2_rows(FAKE, FAKE, 64, 4, tsl.CSA2_FP4_E2M1_E4M3S16)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(k=tsl.csa2_rows(FAKE, None, 128, 1, tsl.CSA2_FP8_E4M3)), tsl.CSA2_ERR_INVALID_ARG),
    (dict(k=tsl.csa2_rows(FAKE, FAKE, 256, 8, tsl.CSA2_FP4_E2M1)), tsl.CSA2_ERR_UNSUPPORTED),
])
def test_cache_write_rejects(kw, status):
    st, msg = _cw(tsl.load(), **kw)
    assert st == status, msg
    assert msg.startswith("csa2_cache_write")


def test_cache_write_zero_tokens_is_a_no_op_after_checks():
    lib = tsl.load()
    assert _cw(lib, T=0)[0] == tsl.CSA2_OK
    # every output format passes the same checks
    for main, k in [(tsl.csa2_rows(FAKE, None, 2048, 0, tsl.CSA2_F32),
                     tsl.csa2_rows(FAKE, None, 512, 0, tsl.CSA2_F32)),
                    (tsl.csa2_rows(FAKE, FAKE + 256, 288, 288, tsl.CSA2_FP4_E2M1_E4M3S16),
                     tsl.csa2_rows(FAKE, FAKE + 4096, 64, 8, tsl.CSA2_FP4_E2M1_E4M3S16)),
                    (None, tsl.csa2_rows(FAKE, FAKE + 8192, 128, 1, tsl.CSA2_FP8_E4M3))]:
        assert _cw(lib, T=0, main=main, k=k)[0] == tsl.CSA2_OK, lib.csa2_last_error()
    # ratio 1 needs neither gates nor a pending row
    assert _cw(lib, T=0, ratio=1, z=None, pend=None)[0] == tsl.CSA2_OK


def test_page_table_checks():
    lib = tsl.load()
    good = tsl.csa2_pages(FAKE, 16, 100, 8448, FAKE)
    # index scores: seq_base may be NULL with pages; the table, its width, the
    # pool size and a 16-byte page stride are required
    st, msg = _scores(lib, Q=0, seq_base=None, pages=good)
    assert st == tsl.CSA2_OK, msg
    assert _scores(lib, seq_base=None)[0] == tsl.CSA2_ERR_INVALID_ARG
    for bad in (tsl.csa2_pages(None, 16, 100, 8448, None), tsl.csa2_pages(FAKE, 0, 100, 8448, None),
                tsl.csa2_pages(FAKE, 16, 0, 8448, None), tsl.csa2_pages(FAKE, 16, 100, 8440, None),
                tsl.csa2_pages(FAKE, 16, 100, -16, None)):
        st, msg = _scores(lib, pages=bad)
        assert st == tsl.CSA2_ERR_INVALID_ARG and "pages" in msg
    # top-k: the table and the row sequences are required
    pp = ctypes.byref
    assert lib.csa2_topk(FAKE, 64, 64, FAKE, 1, None, 0, 8, 8, FAKE, None, 0, 0, pp(good), None) == \
        tsl.CSA2_OK
    assert lib.csa2_topk(FAKE, 64, 64, FAKE, 1, None, 0, 8, 8, FAKE, None, 0, 1,
                         pp(tsl.csa2_pages(FAKE, 16, 0, 0, None)), None) == tsl.CSA2_ERR_INVALID_ARG
    f = lib.csa2_topk_and_block_candidates
    assert f(FAKE, 64, 64, None, 0, FAKE, 1, 8, FAKE, 8, 16, FAKE, None, 0, 1,
             pp(tsl.csa2_pages(None, 16, 0, 0, FAKE)), None) == tsl.CSA2_ERR_INVALID_ARG
