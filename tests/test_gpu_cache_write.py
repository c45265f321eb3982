"""GPU parity of the Full-layer cache write (csa2_cache_write) against the
oracle: main-KV entries and index keys in every output format, the m = 2
pending-row bookkeeping, skip rules, and sampled entries of the 65,536-token
m = 2 prefill chunk.

Tolerance (derived from the kernel's arithmetic): inputs are bf16 and exact
in both; the kernel's softmax weights, sums of squares and norms are fp32
(relative error about 1e-6), and the projection takes the latent as bf16
hi + lo (16 significant bits) times bf16 weights, exact products summed in
fp32 (relative error about 2^-17 per term).  Values before quantization must
agree within 1e-4 of their row's RMS.  A quantized code must be the nearest
code, under the GPU's own scale, of some value within that distance of the
oracle's; fp32 scales must agree within the same distance over fmax, and an
E4M3 scale byte must be the rounding of some amax within it."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_long_amd as tsl

pytestmark = pytest.mark.gpu

TOL = 1e-4
SENTINEL = 0xA5


def _main_buf(fmt, n, dev):
    width = {"f32": 2048, "fp4": 320, "fp4s16": 288}[fmt]
    buf = torch.full((n, width), SENTINEL, dtype=torch.uint8, device=dev)
    if fmt == "f32":
        rows = tsl.csa2_rows(buf.data_ptr(), None, 2048, 0, tsl.CSA2_F32)
    elif fmt == "fp4":
        rows = tsl.rows_fp4_records(buf)
    else:
        rows = tsl.rows_fp4s16_records(buf)
    return buf, rows


def _k_buf(fmt, n, dev):
    if fmt == "f32":
        buf = torch.full((n, 512), SENTINEL, dtype=torch.uint8, device=dev)
        return (buf,), tsl.csa2_rows(buf.data_ptr(), None, 512, 0, tsl.CSA2_F32)
    if fmt == "fp8":
        codes = torch.full((n, 128), SENTINEL, dtype=torch.uint8, device=dev)
        scale = torch.full((n, 4), SENTINEL, dtype=torch.uint8, device=dev)
        return (codes, scale), tsl.csa2_rows(codes.data_ptr(), scale.data_ptr(), 128, 1,
                                             tsl.CSA2_FP8_E4M3)
    codes = torch.full((n, 64), SENTINEL, dtype=torch.uint8, device=dev)
    scales = torch.full((n, 8), SENTINEL, dtype=torch.uint8, device=dev)
    return (codes, scales), tsl.rows_fp4s16(codes, scales)


def run_gpu(inp, main_fmt, k_fmt, main_base, n_main, k_base, n_k, pend=None):
    dev = inp.c.device
    mbuf, mrows = (None, None) if main_fmt is None else _main_buf(main_fmt, n_main, dev)
    kbufs, krows = ((), None) if k_fmt is None else _k_buf(k_fmt, n_k, dev)
    mb = torch.tensor(main_base, dtype=torch.int64, device=dev)
    kb = torch.tensor(k_base, dtype=torch.int64, device=dev)
    tsl.csa2_cache_write(inp.c, inp.z if inp.ratio == 2 else None, inp.tok_seq, inp.tok_pos,
                         inp.ratio, pend, inp.n_seq, inp.kv_norm_w, inp.w_ik, inp.k_norm_w,
                         inp.eps, inp.rope_cs, mrows, mb, n_main, krows, kb, n_k)
    torch.cuda.synchronize()
    return (None if mbuf is None else mbuf.cpu().numpy()), [b.cpu().numpy() for b in kbufs]


def run_oracle(inp, pend, idx=None):
    """The oracle on every token, or (idx) on the listed tokens with their
    pair partners, which must be the previous rows."""
    dec = oracle.decode_bf16
    seq = inp.tok_seq.cpu().numpy()
    pos = inp.tok_pos.cpu().numpy()
    c_all, z_all = inp.c.cpu(), inp.z.cpu()
    if idx is not None:
        rows = sorted(set(int(t) for i in idx for t in range(i - inp.ratio + 1, i + 1)))
        seq, pos = seq[rows], pos[rows]
        c = dec(c_all[rows].numpy())
        z = dec(z_all[rows].numpy())
    else:
        c, z = dec(c_all.numpy()), dec(z_all.numpy())
    pc = pz = None
    if pend is not None:
        p = pend.cpu().numpy()
        pc, pz = dec(p[:, 0]), dec(p[:, 1])
    rope = inp.rope_cs.cpu().double().numpy()
    return oracle.cache_write(c, z, seq, pos, inp.ratio, inp.n_seq, pc, pz,
                              inp.kv_norm_w.cpu().double().numpy(), dec(inp.w_ik.cpu().numpy()),
                              inp.k_norm_w.cpu().double().numpy(), inp.eps,
                              rope[:, :32], rope[:, 32:])


# --------------------------------------------------------------------------
# comparison helpers

def _unpack_e2m1(b):
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def _check_codes(v, codes, scale, kind, tol):
    """v [n, d] oracle values, codes [n, d] GPU codes, scale [n, d] the GPU's
    decoded scale per element, tol [n, 1] allowed distance before quantizing."""
    enc, table = ((oracle.encode_e2m1, oracle.E2M1_TABLE) if kind == "e2m1"
                  else (oracle.encode_e4m3, oracle.E4M3_TABLE))
    y, d = v / scale, tol / scale
    lo, hi = table[enc(y - d)], table[enc(y + d)]
    got = table[codes]
    bad = ~((got >= lo) & (got <= hi))
    assert not bad.any(), (f"{bad.sum()} codes off: first at {np.argwhere(bad)[0]}, "
                           f"value {v[bad][0]}, scale {scale[bad][0]}, code {codes[bad][0]}")
    return float(np.mean(codes == enc(y)))


def _check_fp32_scales(v, scale, group, fmax, tol):
    amax = np.abs(v).reshape(len(v), -1, group).max(axis=2)
    want = np.where(amax > 0, amax / fmax, 1.0)
    assert np.all(np.abs(scale - want) <= tol / fmax + 1e-6 * want), np.max(np.abs(scale - want))


def _check_s16_scales(v, sbytes, tol):
    amax = np.abs(v).reshape(len(v), -1, 16).max(axis=2)

    def val(a):          # the scale value the rule gives an amax a > 0
        b = oracle.encode_e4m3(a / 6.0)
        return oracle.E4M3_TABLE[np.where(b == 0, 0x01, b)]
    got = oracle.E4M3_TABLE[sbytes]
    ok = (got >= val(np.maximum(amax - tol, 1e-30))) & (got <= val(amax + tol))
    ok |= (amax <= tol) & (sbytes == 0x38)     # an all-zero group takes 1.0
    assert ok.all()


def check_main(fmt, rows_gpu, v):
    tol = TOL * np.sqrt(np.mean(v * v, axis=1, keepdims=True))
    if fmt == "f32":
        got = rows_gpu.view("<f4").astype(np.float64)
        assert np.all(np.abs(got - v) <= tol), np.max(np.abs(got - v) / tol)
        return 1.0
    codes = _unpack_e2m1(rows_gpu[:, :256])
    if fmt == "fp4":
        scale = rows_gpu[:, 256:320].copy().view("<f4").astype(np.float64)
        _check_fp32_scales(v, scale, 32, 6.0, tol)
        return _check_codes(v, codes, np.repeat(scale, 32, axis=1), "e2m1", tol)
    sb = rows_gpu[:, 256:288]
    _check_s16_scales(v, sb, tol)
    return _check_codes(v, codes, np.repeat(oracle.E4M3_TABLE[sb], 16, axis=1), "e2m1", tol)


def check_k(fmt, bufs, rows, v):
    tol = TOL * np.sqrt(np.mean(v * v, axis=1, keepdims=True))
    if fmt == "f32":
        got = bufs[0][rows].copy().view("<f4").astype(np.float64)
        assert np.all(np.abs(got - v) <= tol), np.max(np.abs(got - v) / tol)
        return 1.0
    if fmt == "fp8":
        codes = bufs[0][rows]
        scale = bufs[1][rows].copy().view("<f4").astype(np.float64)      # [n, 1]
        _check_fp32_scales(v, scale, 128, 448.0, tol)
        return _check_codes(v, codes, np.repeat(scale, 128, axis=1), "e4m3", tol)
    codes = _unpack_e2m1(bufs[0][rows])
    sb = bufs[1][rows]
    _check_s16_scales(v, sb, tol)
    return _check_codes(v, codes, np.repeat(oracle.E4M3_TABLE[sb], 16, axis=1), "e2m1", tol)


def _bases(inp, cap_per_seq):
    return [s * cap_per_seq for s in range(inp.n_seq)]


def _compare(inp, main_fmt, k_fmt, pend, cap, main_base=None, k_base=None, n_main=None,
             n_k=None):
    main_base = _bases(inp, cap) if main_base is None else main_base
    k_base = _bases(inp, cap) if k_base is None else k_base
    n_main = inp.n_seq * cap if n_main is None else n_main
    n_k = inp.n_seq * cap if n_k is None else n_k
    pend_gpu = None if pend is None else pend.clone()
    mg, kg = run_gpu(inp, main_fmt, k_fmt, main_base, n_main, k_base, n_k, pend_gpu)
    ent, mo, ko, pc, pz = run_oracle(inp, pend)
    mrow = np.array([main_base[s] + e for s, e in ent], dtype=np.int64)
    krow = np.array([k_base[s] + e for s, e in ent], dtype=np.int64)
    mok = (mrow >= 0) & (mrow < n_main)
    kok = (krow >= 0) & (krow < n_k)
    exact = []
    if main_fmt is not None:
        exact.append(check_main(main_fmt, mg[mrow[mok]], mo[mok]))
        untouched = np.ones(n_main, dtype=bool)
        untouched[mrow[mok]] = False
        assert np.all(mg[untouched] == SENTINEL)
    if k_fmt is not None:
        exact.append(check_k(k_fmt, kg, krow[kok], ko[kok]))
        untouched = np.ones(n_k, dtype=bool)
        untouched[krow[kok]] = False
        assert all(np.all(b[untouched] == SENTINEL) for b in kg)
    if pend is not None:
        got = pend_gpu.cpu().numpy()
        assert np.array_equal(oracle.decode_bf16(got[:, 0]), pc)
        assert np.array_equal(oracle.decode_bf16(got[:, 1]), pz)
    return ent, exact


FORMATS = [("f32", "f32"), ("fp4", "fp8"), ("fp4s16", "fp4s16")]


@pytest.mark.parametrize("ratio", [1, 2])
@pytest.mark.parametrize("main_fmt,k_fmt", FORMATS)
def test_cache_write_mixed_batch(ratio, main_fmt, k_fmt):
    """Several sequences with odd and even starts, a ragged tail, a run past
    the RoPE table, a sequence id out of range and rows past the capacity."""
    runs = [(0, 0, 150), (1, 7, 33), (2, 1000, 3), (3, 64, 64), (4, 5, 2), (5, 20, 9)]
    inp = synth.cache_write_inputs(31 + ratio, runs, ratio, "cuda", n_seq=5, n_rope=900)
    print(f"cache write mixed batch: ratio {ratio}, {main_fmt}/{k_fmt}, T {inp.c.shape[0]}",
          flush=True)
    cap = 600
    main_base = [0, 600, 1200, 1800, 2998]     # sequence 4's main rows fall past 3000
    ent, exact = _compare(inp, main_fmt, k_fmt, inp.pend, cap, main_base=main_base,
                          n_main=3000)
    assert len(ent) > 100 // ratio
    assert all(s != 5 for s, _ in ent) and all(s != 2 for s, _ in ent)
    assert any(s == 4 for s, _ in ent)         # its index keys are still written
    assert min(exact) > 0.99


@pytest.mark.parametrize("ratio", [1, 2])
def test_cache_write_main_only_and_keys_only(ratio):
    runs = [(0, 3, 70), (1, 0, 41)]
    inp = synth.cache_write_inputs(40 + ratio, runs, ratio, "cuda")
    _compare(inp, "fp4", None, inp.pend, 128)
    _compare(inp, None, "fp8", inp.pend, 128)


def test_cache_write_without_pending_rows():
    """Without pend, a run that starts at an odd position drops its first
    token; nothing else changes."""
    runs = [(0, 1, 10), (1, 0, 10)]
    inp = synth.cache_write_inputs(50, runs, 2, "cuda", with_pend=False)
    ent, _ = _compare(inp, "fp4", "fp8", None, 16)
    assert (0, 0) not in ent and (0, 1) in ent and len(ent) == 4 + 5


def test_cache_write_decode_batch_pairs():
    """One token per sequence, 64 sequences at mixed positions: every odd one
    closes a pair with its pending row (up to 64 entries in one workgroup)."""
    rng = np.random.default_rng(51)
    pos = rng.integers(0, 4000, size=64)
    pos[:40] |= 1                          # at least 40 closing tokens
    runs = [(s, int(p), 1) for s, p in enumerate(pos)]
    inp = synth.cache_write_inputs(52, runs, 2, "cuda")
    ent, exact = _compare(inp, "fp4s16", "fp4s16", inp.pend, 2048)
    assert len(ent) == int(np.sum(pos % 2 == 1))


def test_cache_write_chunked_calls_equal_one_call():
    """A sequence written over several calls (odd and even split points, the
    pending row carried) gets the same bytes as one call."""
    runs = [(0, 0, 301)]
    whole = synth.cache_write_inputs(60, runs, 2, "cuda")
    pend0 = whole.pend.clone()
    mg, kg = run_gpu(whole, "fp4", "fp8", [0], 256, [0], 256, pend0.clone())
    pend = pend0.clone()
    parts_m, parts_k = [], []
    for lo, hi in [(0, 3), (3, 4), (4, 131), (131, 200), (200, 301)]:
        part = synth.CacheWriteInputs(**{**whole.__dict__, "c": whole.c[lo:hi].contiguous(),
                                         "z": whole.z[lo:hi].contiguous(),
                                         "tok_seq": whole.tok_seq[lo:hi].contiguous(),
                                         "tok_pos": whole.tok_pos[lo:hi].contiguous()})
        m_, k_ = run_gpu(part, "fp4", "fp8", [0], 256, [0], 256, pend)
        parts_m.append(m_)
        parts_k.append(k_)
    # every entry was written by exactly one of the calls
    merged = np.full_like(mg, SENTINEL)
    for m_ in parts_m:
        w = np.any(m_ != SENTINEL, axis=1)
        assert not np.any(np.any(merged[w] != SENTINEL, axis=1))
        merged[w] = m_[w]
    assert np.array_equal(merged, mg)
    mk = [np.full_like(b, SENTINEL) for b in kg]
    for k_ in parts_k:
        w = np.any(k_[0] != SENTINEL, axis=1)
        for dst, src in zip(mk, k_):
            dst[w] = src[w]
    assert all(np.array_equal(a, b) for a, b in zip(mk, kg))
    # token 300 opened a pair that no call closed
    assert torch.equal(pend[0, 0], whole.c[300]) and torch.equal(pend[0, 1], whole.z[300])


def test_cache_write_prefill_chunk_sampled():
    """The encoder Full layer's 65,536-token m = 2 chunk (32,768 entries), in
    the bench's formats; 256 sampled entries against the oracle, and every
    entry row written."""
    T = 65536
    inp = synth.cache_write_inputs(2, [(0, 0, T)], 2, "cuda")
    print("cache write prefill chunk: 65536 tokens, m = 2", flush=True)
    n = T // 2
    mg, kg = run_gpu(inp, "fp4", "fp8", [0], n, [0], n, inp.pend.clone())
    assert not np.any(np.all(mg == SENTINEL, axis=1))
    assert not np.any(np.all(kg[0] == SENTINEL, axis=1))
    rng = np.random.default_rng(3)
    # random entries, plus a tile edge and the last entry
    ents = np.array(sorted(set(rng.choice(n, size=256, replace=False).tolist()) | {31, n - 1}))
    ent, mo, ko, _, _ = run_oracle(inp, None, idx=[2 * e + 1 for e in ents])
    assert [e for _, e in ent] == list(ents)
    assert check_main("fp4", mg[ents], mo) > 0.99
    assert check_k("fp8", kg, ents, ko) > 0.99
