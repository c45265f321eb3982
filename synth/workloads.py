"""Seeded synthetic workloads shaped like the pages' CSA2 configurations.

Each workload is a set of device-resident tensors plus the metadata the four
library calls need.  Nothing here scores, selects or attends: the tensors are
random draws, encoded into the cache formats by :mod:`synth.formats`.

The shapes follow the V4.1-Flash description (CSA2 deep-dive page, sections on
the per-layer attention computation, the hierarchical sparse indexer and the
V4.1-Flash layout; V4.1-Flash report reading, sections 4 and 5):

* indexer 32 heads x 128 dims, top-512, 8-position blocks, 2048 kept blocks;
* attention 64 heads x 512 dims, MQA with K = V, 128 sliding-window entries;
* decoder ratio m = 1, encoder ratio m = 2 (per-channel softmax pooling of
  non-overlapping token pairs, no positional bias).

Random streams: every tensor draws from its own torch.Generator seeded with a
64-bit value derived by numpy's SeedSequence from (seed, tensor id, chunk), so
a tensor never depends on which other tensors were drawn.  Large tensors are
drawn in fixed chunks of 2^20 rows so the values do not depend on the memory
available.  The same seed gives the same bytes on the same device type; CPU
and GPU draws differ (different generators), and each test uses one device's
draw for both sides of a comparison.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

from .formats import (encode_e4m3_rows, encode_fp4_records, encode_fp4s16_rows,
                      encode_fp4s16_records, encode_swa_records,
                      encode_bf16)

CONFIG_NAMES = ("tiny_full_fp32", "decode_128k", "prefill_m2_chunk",
                "reindex_1m", "decoder_group_256k")
# further workloads of the same shapes in other cache formats
EXTRA_WORKLOADS = ("decode_128k_pages_formats",)

H_IDX, D_IDX = 32, 128
H_ATT, D_ATT = 64, 512
TOPK, BLOCK, N_BLOCKS, WINDOW = 512, 8, 2048, 128
CHUNK_ROWS = 1 << 20

# tensor ids for the seed derivation
_T_KIDX, _T_MAIN, _T_C, _T_Z = 1, 2, 3, 4
_T_QIDX, _T_W, _T_Q, _T_SWA, _T_SINK = 10, 11, 12, 13, 14
_T_CW_C, _T_CW_Z, _T_CW_KVW, _T_CW_KW, _T_CW_WIK, _T_CW_PEND = 20, 21, 22, 23, 24, 25


def _gen(seed, tid, sub, device):
    s = np.random.SeedSequence([int(seed), int(tid), int(sub)])
    v = int(s.generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(v)
    return g


def _randn(shape, seed, tid, sub, device):
    return torch.randn(shape, generator=_gen(seed, tid, sub, device),
                       device=device, dtype=torch.float32)


def _randint(lo, hi, shape, seed, tid, sub, device):
    """Integers uniform in [lo, hi], as fp32."""
    return torch.randint(lo, hi + 1, shape, generator=_gen(seed, tid, sub, device),
                         device=device).to(torch.float32)


@dataclass
class Layer:
    mode: str                      # "full", "reindex" or "reuse"
    q: torch.Tensor                # [Q, H, D] bf16 bits (int16) or fp32
    swa: torch.Tensor              # [rows, 528] u8 records, or [rows, 512] fp32
    sink: torch.Tensor             # [H] fp32
    q_idx: torch.Tensor = None     # [Q, 32, 128] u8 E4M3 codes, or fp32
    q_scale: torch.Tensor = None   # [Q, 32] fp32 (None for fp32 q_idx)
    w: torch.Tensor = None         # [Q, 32] bf16 bits (int16), or fp32


@dataclass
class Workload:
    name: str
    seed: int
    quantized: bool
    ratio: int
    n_entries: list                # main-KV / index-K entries per sequence
    seq_base: torch.Tensor         # [B] int64 first row of each sequence
    q_seq: torch.Tensor            # [Q] int32
    q_pos: torch.Tensor            # [Q] int32 token position of each query
    k_idx: torch.Tensor            # [sum N, 128] u8 E4M3 codes ([sum N, 64] E2M1 pairs), or fp32
    k_scale: torch.Tensor          # [sum N] fp32 ([sum N, 8] u8 E4M3 for E2M1 keys), or None
    main_kv: torch.Tensor          # [sum N, 320] u8 records ([sum N, 288] for "fp4s16"), or fp32
    swa_base: torch.Tensor         # [B] int64 first SWA row of each sequence
    swa_pos0: torch.Tensor         # [B] int32 token position of that row
    layers: list = field(default_factory=list)
    topk: int = TOPK
    block_size: int = BLOCK
    n_blocks: int = N_BLOCKS
    window: int = WINDOW
    softmax_scale: float = 1.0 / math.sqrt(D_ATT)
    k_fmt: str = "fp8"             # index-K format: "fp8" (E4M3 + fp32 per row) or "fp4s16"
    main_fmt: str = "fp4"          # main-KV record: "fp4" (320 B, fp32 per 32) or "fp4s16" (288 B)

    @property
    def Q(self):
        return int(self.q_pos.shape[0])

    @property
    def B(self):
        return len(self.n_entries)

    def n_vis(self):
        """Visible main entries per query: (pos + 1) // ratio."""
        return (self.q_pos.to(torch.int64) + 1) // self.ratio

    def max_cols(self):
        return int(self.n_vis().max().item())

    def to(self, device):
        """Copy every tensor to `device` (the values do not change)."""
        def mv(x):
            return None if x is None else x.to(device)
        out = Workload(**{f: getattr(self, f) for f in self.__dataclass_fields__})
        for f in ("seq_base", "q_seq", "q_pos", "k_idx", "k_scale", "main_kv", "swa_base",
                  "swa_pos0"):
            setattr(out, f, mv(getattr(self, f)))
        out.layers = [Layer(mode=l.mode, q=mv(l.q), swa=mv(l.swa), sink=mv(l.sink),
                            q_idx=mv(l.q_idx), q_scale=mv(l.q_scale), w=mv(l.w))
                      for l in self.layers]
        return out


def _chunked(total, fn):
    parts = []
    for c, r0 in enumerate(range(0, total, CHUNK_ROWS)):
        parts.append(fn(c, min(CHUNK_ROWS, total - r0)))
    return torch.cat(parts, 0) if len(parts) > 1 else parts[0]


def _index_keys(seed, total, quantized, device, k_fmt="fp8"):
    if not quantized:
        return _randint(-4, 4, (total, D_IDX), seed, _T_KIDX, 0, device), None
    enc = encode_fp4s16_rows if k_fmt == "fp4s16" else encode_e4m3_rows

    def one(c, n):
        return enc(_randn((n, D_IDX), seed, _T_KIDX, c, device))
    parts = []
    for c, r0 in enumerate(range(0, total, CHUNK_ROWS)):
        parts.append(one(c, min(CHUNK_ROWS, total - r0)))
    codes = torch.cat([p[0] for p in parts], 0)
    scale = torch.cat([p[1] for p in parts], 0)
    if k_fmt != "fp4s16":
        scale = scale.reshape(total)
    return codes, scale


def _main_kv_gauss(seed, total, quantized, device, main_fmt="fp4"):
    if not quantized:
        return _randn((total, D_ATT), seed, _T_MAIN, 0, device)
    enc = encode_fp4s16_records if main_fmt == "fp4s16" else encode_fp4_records
    return _chunked(total, lambda c, n: enc(_randn((n, D_ATT), seed, _T_MAIN, c, device)))


def compress_pairs_input(c, z):
    """Input recipe for the m = 2 encoder cache: entry i, channel ch is the
    softmax over the token pair (2i, 2i+1) of the logits z, applied to c
    (V4.1 report reading section 4 and the xhh.club summary: non-overlapping
    groups, per-channel softmax, no positional bias)."""
    n = c.shape[0] // 2
    c2 = c[: 2 * n].reshape(n, 2, -1)
    z2 = z[: 2 * n].reshape(n, 2, -1)
    wgt = torch.softmax(z2, dim=1)
    return (wgt * c2).sum(dim=1)


def _layer(seed, li, mode, Q, swa_rows, quantized, device, with_indexer):
    base = 100 * (li + 1)
    if quantized:
        q = encode_bf16(_randn((Q, H_ATT, D_ATT), seed, _T_Q + base, 0, device))
        swa = encode_swa_records(_randn((swa_rows, D_ATT), seed, _T_SWA + base, 0, device))
    else:
        q = _randn((Q, H_ATT, D_ATT), seed, _T_Q + base, 0, device)
        swa = _randn((swa_rows, D_ATT), seed, _T_SWA + base, 0, device)
    sink = _randn((H_ATT,), seed, _T_SINK + base, 0, device)
    lay = Layer(mode=mode, q=q, swa=swa, sink=sink)
    if with_indexer:
        if quantized:
            x = _randn((Q * H_IDX, D_IDX), seed, _T_QIDX + base, 0, device)
            codes, sc = encode_e4m3_rows(x)
            lay.q_idx = codes.reshape(Q, H_IDX, D_IDX)
            lay.q_scale = sc.reshape(Q, H_IDX)
            lay.w = encode_bf16(_randn((Q, H_IDX), seed, _T_W + base, 0, device))
        else:
            lay.q_idx = _randint(-4, 4, (Q, H_IDX, D_IDX), seed, _T_QIDX + base, 0, device)
            lay.w = _randint(-2, 2, (Q, H_IDX), seed, _T_W + base, 0, device)
    return lay


def _decode_layout(n_entries, q_per_seq, ratio, device, positions=None):
    """Decode-style layout: sequence b holds n_entries[b] entries; its queries
    sit at the end of the sequence (or at explicit positions)."""
    B = len(n_entries)
    seq_base = torch.tensor(np.concatenate([[0], np.cumsum(n_entries)[:-1]]),
                            dtype=torch.int64)
    q_seq, q_pos = [], []
    for b in range(B):
        if positions is not None:
            ps = positions[b]
        else:
            last = n_entries[b] * ratio - 1
            ps = [last - i for i in range(q_per_seq)]
        q_seq += [b] * len(ps)
        q_pos += list(ps)
    q_seq = torch.tensor(q_seq, dtype=torch.int32)
    q_pos = torch.tensor(q_pos, dtype=torch.int32)
    # SWA rows cover [min pos - window + 1, max pos] of each sequence
    swa_pos0, swa_rows = [], []
    for b in range(B):
        ps = q_pos[q_seq == b]
        lo = max(0, int(ps.min()) - WINDOW + 1) if len(ps) else 0
        hi = int(ps.max()) if len(ps) else -1
        swa_pos0.append(lo)
        swa_rows.append(max(0, hi - lo + 1))
    swa_base = torch.tensor(np.concatenate([[0], np.cumsum(swa_rows)[:-1]]),
                            dtype=torch.int64)
    return (seq_base.to(device), q_seq.to(device), q_pos.to(device),
            swa_base.to(device), torch.tensor(swa_pos0, dtype=torch.int32).to(device),
            int(sum(swa_rows)))


def mini_workload(seed, n_entries, q_per_seq=1, ratio=1, quantized=True,
                  modes=("full",), device="cpu", positions=None, topk=TOPK,
                  n_blocks=N_BLOCKS, block_size=BLOCK, k_fmt="fp8", main_fmt="fp4"):
    """A small workload of the same structure, for parity tests."""
    seq_base, q_seq, q_pos, swa_base, swa_pos0, swa_total = _decode_layout(
        n_entries, q_per_seq, ratio, device, positions)
    total = int(sum(n_entries))
    k_idx, k_scale = _index_keys(seed, total, quantized, device, k_fmt)
    main = _main_kv_gauss(seed, total, quantized, device, main_fmt)
    Q = int(q_pos.shape[0])
    layers = [_layer(seed, li, m, Q, swa_total, quantized, device,
                     with_indexer=(m in ("full", "reindex")))
              for li, m in enumerate(modes)]
    return Workload(name="mini", seed=seed, quantized=quantized, ratio=ratio,
                    n_entries=list(n_entries), seq_base=seq_base, q_seq=q_seq,
                    q_pos=q_pos, k_idx=k_idx, k_scale=k_scale, main_kv=main,
                    swa_base=swa_base, swa_pos0=swa_pos0, layers=layers,
                    topk=topk, n_blocks=n_blocks, block_size=block_size,
                    k_fmt=k_fmt if quantized else "fp8",
                    main_fmt=main_fmt if quantized else "fp4")


def _prefill_m2(seed, device):
    """Encoder Full-layer prefill chunk: 65,536 tokens compressed in pairs to
    32,768 entries; 4,096 causal queries at the end of the sequence."""
    n_tok, n_q = 65536, 4096
    n_ent = n_tok // 2
    main_parts = []
    for c, r0 in enumerate(range(0, n_ent, CHUNK_ROWS // 2)):
        n = min(CHUNK_ROWS // 2, n_ent - r0)
        cc = _randn((2 * n, D_ATT), seed, _T_C, c, device)
        zz = _randn((2 * n, D_ATT), seed, _T_Z, c, device)
        main_parts.append(encode_fp4_records(compress_pairs_input(cc, zz)))
    main = torch.cat(main_parts, 0)
    k_idx, k_scale = _index_keys(seed, n_ent, True, device)
    positions = [list(range(n_tok - n_q, n_tok))]
    seq_base, q_seq, q_pos, swa_base, swa_pos0, swa_total = _decode_layout(
        [n_ent], None, 2, device, positions)
    layers = [_layer(seed, 0, "full", n_q, swa_total, True, device, True)]
    return Workload(name="prefill_m2_chunk", seed=seed, quantized=True, ratio=2,
                    n_entries=[n_ent], seq_base=seq_base, q_seq=q_seq, q_pos=q_pos,
                    k_idx=k_idx, k_scale=k_scale, main_kv=main, swa_base=swa_base,
                    swa_pos0=swa_pos0, layers=layers)


def make_workload(name, device="cpu", seed_offset=0):
    """The five configurations, by name (see CONFIG_NAMES).  seed_offset
    draws an independent copy of the same shapes."""
    o = seed_offset
    if name == "tiny_full_fp32":
        w = mini_workload(0 + o, [2048], q_per_seq=16, ratio=1, quantized=False,
                          modes=("full",), device=device)
    elif name == "decode_128k":
        # Full layer at 128K, batch 8; a Reindex layer on the same cache
        # exercises pool scoring at the same context.
        w = mini_workload(1 + o, [131072] * 8, q_per_seq=1, ratio=1, quantized=True,
                          modes=("full", "reindex"), device=device)
    elif name == "prefill_m2_chunk":
        w = _prefill_m2(2 + o, device)
    elif name == "decode_128k_pages_formats":
        # decode_128k in the pages' own cache formats: index K as E2M1 with an
        # E4M3 scale per 16 dims (72 B per key instead of 132) and the 288-B
        # main-KV record (instead of 320)
        w = mini_workload(1 + o, [131072] * 8, q_per_seq=1, ratio=1, quantized=True,
                          modes=("full", "reindex"), device=device, k_fmt="fp4s16",
                          main_fmt="fp4s16")
    elif name == "reindex_1m":
        w = mini_workload(3 + o, [1 << 20] * 2, q_per_seq=1, ratio=1, quantized=True,
                          modes=("full", "reindex"), device=device)
    elif name == "decoder_group_256k":
        w = mini_workload(4 + o, [262144] * 64, q_per_seq=1, ratio=1, quantized=True,
                          modes=("full", "reuse", "reuse", "reuse",
                                 "reindex", "reuse", "reuse", "reuse"),
                          device=device)
    else:
        raise ValueError(f"unknown workload {name!r}; known: {CONFIG_NAMES + EXTRA_WORKLOADS}")
    w.name = name
    return w


# ---------------------------------------------------------------------------
# Inputs of the Full-layer cache write

@dataclass
class CacheWriteInputs:
    """Token rows and parameters of one cache-write call.  c, z: bf16 [T, 512]
    compressor projections (z: gate logits); tok_seq, tok_pos: int32 [T];
    pend: bf16 [B, 2, 512] pending rows (or None); kv_norm_w [512] and
    k_norm_w [128] fp32 RMSNorm weights; w_ik bf16 [128, 512]; rope_cs fp32
    [n_rope, 64] (cos of the 32 angles of each position, then their sin)."""
    c: torch.Tensor
    z: torch.Tensor
    tok_seq: torch.Tensor
    tok_pos: torch.Tensor
    ratio: int
    n_seq: int
    pend: torch.Tensor
    kv_norm_w: torch.Tensor
    k_norm_w: torch.Tensor
    w_ik: torch.Tensor
    rope_cs: torch.Tensor
    eps: float = 1e-6


def rope_table(n_pos, device, base=10000.0):
    """cos / sin of position p times the 32 frequencies base^(-2i/64), the
    usual rotary table for 64 rotated dims (drawn in float64, stored fp32)."""
    f = base ** (-torch.arange(32, dtype=torch.float64) * 2.0 / 64.0)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * f[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], 1).to(torch.float32).to(device).contiguous()


def cache_write_inputs(seed, runs, ratio, device, n_seq=None, with_pend=True, n_rope=None):
    """runs: list of (seq, first_position, n_tokens), one run of consecutive
    positions per sequence, in call order.  c and z are N(0, 1) draws
    rounded to bf16; the RMSNorm weights are 1 + N(0, 0.1^2) (the report
    reading's section 6 puts the weights' magnitude near 1); W_IK is
    N(0, 1/512), so index keys have unit scale before their norm; the pending
    rows are N(0, 1) bf16 draws."""
    seq = torch.cat([torch.full((n,), s, dtype=torch.int32) for s, _, n in runs])
    pos = torch.cat([torch.arange(p0, p0 + n, dtype=torch.int32) for _, p0, n in runs])
    T = int(seq.numel())
    n_seq = (max(s for s, _, _ in runs) + 1) if n_seq is None else n_seq
    rows = []
    for tid in (_T_CW_C, _T_CW_Z):
        parts = [encode_bf16(_randn((min(CHUNK_ROWS, T - r0), D_ATT), seed, tid, ci, device))
                 for ci, r0 in enumerate(range(0, T, CHUNK_ROWS))]
        rows.append(torch.cat(parts, 0) if parts else
                    torch.empty((0, D_ATT), dtype=torch.bfloat16, device=device))
    pend = None
    if with_pend:
        pend = encode_bf16(_randn((n_seq * 2, D_ATT), seed, _T_CW_PEND, 0, device)).reshape(n_seq, 2, D_ATT)
    kvw = 1.0 + 0.1 * _randn((D_ATT,), seed, _T_CW_KVW, 0, device)
    kw = 1.0 + 0.1 * _randn((D_IDX,), seed, _T_CW_KW, 0, device)
    w_ik = encode_bf16(_randn((D_IDX, D_ATT), seed, _T_CW_WIK, 0, device) / math.sqrt(D_ATT))
    max_pos = max(p0 + n for _, p0, n in runs)
    rope = rope_table(max_pos if n_rope is None else n_rope, device)
    return CacheWriteInputs(c=rows[0].contiguous(), z=rows[1].contiguous(),
                            tok_seq=seq.to(device), tok_pos=pos.to(device), ratio=ratio,
                            n_seq=n_seq, pend=pend, kv_norm_w=kvw.contiguous(),
                            k_norm_w=kw.contiguous(), w_ik=w_ik.contiguous(), rope_cs=rope)


# ---------------------------------------------------------------------------
# Paged serving layout of a workload's caches (DSA page, top-k section and
# implementation notes: 64-slot pages; an index-key page holds its 64 keys and
# then their 64 scales, 8448 B for FP8 keys with fp32 scales)

PAGE_SLOTS = 64


@dataclass
class PagedLayout:
    """page_table int32 [B, pages of the longest sequence] (-1 past a
    sequence's pages); k_pool u8 [n_pages, k_page_bytes]: each page holds
    64 key rows of k_row_bytes, then 64 scale rows of k_scale_row_bytes from
    k_scale_offset; main_pool u8 [n_pages * 64, record bytes] (slot rows);
    rope_cs fp32 [positions, 64]."""
    page_table: torch.Tensor
    n_pages: int
    k_pool: torch.Tensor
    k_page_bytes: int
    k_row_bytes: int
    k_scale_offset: int
    k_scale_row_bytes: int
    main_pool: torch.Tensor
    rope_cs: torch.Tensor


def paged_layout(wl, seed, spare_pages=3):
    """Scatter a quantized workload's index keys and main-KV records into a
    pool of 64-slot pages in a seeded random page order (plus a few pages no
    sequence uses).  Only bytes move; values are the workload's."""
    assert wl.quantized
    dev = wl.k_idx.device
    per = [(n + PAGE_SLOTS - 1) // PAGE_SLOTS for n in wl.n_entries]
    n_pages = sum(per) + spare_pages
    g = torch.Generator()
    g.manual_seed(int(np.random.SeedSequence([int(seed), 90]).generate_state(1, np.uint64)[0]) & ((1 << 63) - 1))
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    table = torch.full((wl.B, max(per)), -1, dtype=torch.int32)
    o = 0
    for b, n in enumerate(per):
        table[b, :n] = perm[o:o + n]
        o += n
    table = table.to(dev)
    fp4 = getattr(wl, "k_fmt", "fp8") == "fp4s16"
    kb = 64 if fp4 else 128
    sb = 8 if fp4 else 4
    page_bytes = PAGE_SLOTS * (kb + sb)
    k_pool = torch.zeros((n_pages, page_bytes), dtype=torch.uint8, device=dev)
    rec = wl.main_kv.shape[1]
    main_pool = torch.zeros((n_pages * PAGE_SLOTS, rec), dtype=torch.uint8, device=dev)
    k_scale_bytes = wl.k_scale.contiguous().view(torch.uint8).reshape(wl.k_idx.shape[0], sb)
    keys = k_pool[:, :PAGE_SLOTS * kb].view(n_pages, PAGE_SLOTS, kb)     # strided views
    scales = k_pool[:, PAGE_SLOTS * kb:].view(n_pages, PAGE_SLOTS, sb)
    for b, n in enumerate(wl.n_entries):
        p = torch.arange(n, device=dev)
        page = table[b, p // PAGE_SLOTS].to(torch.int64)
        slot = p % PAGE_SLOTS
        rows = int(wl.seq_base[b].item()) + p
        keys[page, slot] = wl.k_idx[rows]
        scales[page, slot] = k_scale_bytes[rows]
        main_pool[page * PAGE_SLOTS + slot] = wl.main_kv[rows]
    rope = rope_table(int(wl.q_pos.max().item()) + 1, dev)
    return PagedLayout(page_table=table.contiguous(), n_pages=n_pages, k_pool=k_pool,
                       k_page_bytes=page_bytes, k_row_bytes=kb, k_scale_offset=PAGE_SLOTS * kb,
                       k_scale_row_bytes=sb, main_pool=main_pool, rope_cs=rope)
