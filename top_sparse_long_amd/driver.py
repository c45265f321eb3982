"""Layer driver over the shared slot set (the cross-layer orchestration step).

A decoder group runs its layers in order over one set of slots
(xhh.club three-modes page, "shared pool mechanism": the runtime holds
compress_kv, index_k, topk_idxs and candidates; CSA2 page, "three modes"):

* Full    scores every visible entry, writes topk_idxs and, when a later
          Reindex layer will use it, the candidate pool (CSA2 page,
          "hierarchical sparse indexer");
* Reindex scores only the pool with its own indexer query and rewrites
          topk_idxs (without a pool it scores every visible entry);
* Reuse   runs no indexer and reads topk_idxs.
Every layer brings its own q, SWA rows and sink.  Only device pointers move
between layers; every step is a call into libcsa2.so.

The driver takes any object with the attributes of synth.Workload (the cache
tensors, the per-query metadata and a list of layers).
"""
import math

import torch

from . import (csa2_index_scores, csa2_block_candidates, csa2_topk, csa2_sparse_attn,
               csa2_topk_and_block_candidates, csa2_topk_and_block_candidates_workspace_size,
               csa2_block_candidates_workspace_size, csa2_topk_workspace_size,
               csa2_sparse_attn_workspace_size, csa2_rows, csa2_pages,
               csa2_topk_from_block_max, csa2_topk_from_block_max_workspace_size,
               csa2_top_blocks_and_block_candidates, csa2_top_blocks_and_block_candidates_workspace_size,
               rows_f32, rows_fp8, rows_fp4s16, rows_fp4_records, rows_fp4s16_records,
               rows_swa_records,
               CSA2_F32, CSA2_BF16, CSA2_FP8_E4M3, CSA2_FP4_E2M1_E4M3S16)


# the re-scoring route for a Full layer's top-k (see LayerRunner): measured
# per step, 64 x 262,144 keys 732.9 -> 680.8 us; with the scorer's storing
# wave for maxima-only calls, 2 x 1,048,576 145.1 -> 143.2 us, while
# 8 x 131,072 keys lose (105.5 -> 110.7: the two extra launches cost more
# than the score writes they save)
RESCORE_MAX_Q = 256
RESCORE_MIN_KEYS = 2 << 20


def _round_up(x, m):
    return (x + m - 1) // m * m


class SlotSet:
    """The four cross-layer slots.  compress_kv and index_k are the cache
    row descriptors; topk_idxs and candidates are device tensors."""

    def __init__(self, compress_kv, index_k):
        self.compress_kv = compress_kv
        self.index_k = index_k
        self.topk_idxs = None
        self.candidates = None


class LayerRunner:
    """paged: an optional synth.PagedLayout — index keys are read through its
    page table, the top-k writes physical slots and attention gathers by
    slot; rope_cs: an optional [positions, 64] table — attention turns its
    output back by each query's position (the layout's table when paged)."""

    def __init__(self, wl, device="cuda", paged=None, rope_cs=None, via_blocks=True, rescore=None):
        self.wl = wl
        self.dev = device
        self.paged = paged
        self.rope_cs = paged.rope_cs if (paged is not None and rope_cs is None) else rope_cs
        Q = wl.Q
        self.Q = Q
        self.quant = wl.quantized
        self.n_cols = wl.max_cols()
        self.stride = _round_up(max(self.n_cols, 4), 64)
        self.pool_cols = wl.n_blocks * wl.block_size
        if self.quant:
            if getattr(wl, "k_fmt", "fp8") == "fp4s16":
                self.k_rows = rows_fp4s16(wl.k_idx, wl.k_scale)
            else:
                self.k_rows = rows_fp8(wl.k_idx, wl.k_scale)
            if getattr(wl, "main_fmt", "fp4") == "fp4s16":
                self.main_rows = rows_fp4s16_records(wl.main_kv)
            else:
                self.main_rows = rows_fp4_records(wl.main_kv)
        else:
            self.k_rows = rows_f32(wl.k_idx)
            self.main_rows = rows_f32(wl.main_kv)
        self.layer_rows = []
        for lay in wl.layers:
            d = {}
            if self.quant:
                d["swa"] = rows_swa_records(lay.swa)
                if lay.q_idx is not None:
                    d["q_idx"] = rows_fp8(lay.q_idx.reshape(Q * 32, 128), lay.q_scale.reshape(Q * 32))
            else:
                d["swa"] = rows_f32(lay.swa)
                if lay.q_idx is not None:
                    d["q_idx"] = rows_f32(lay.q_idx.reshape(Q * 32, 128))
            self.layer_rows.append(d)
        self.needs_pool = [any(l.mode == "reindex" for l in wl.layers[i + 1:])
                           for i in range(len(wl.layers))]
        f32 = torch.float32
        self.scores = torch.empty((Q, self.stride), dtype=f32, device=device)
        # block maxima written by the Full layer's scoring pass
        self.fuse_block_max = wl.block_size <= 32
        # a Full layer's top-k ranks blocks by those maxima first
        self.via_blocks = via_blocks and self.fuse_block_max
        nbm = (self.n_cols + wl.block_size - 1) // wl.block_size
        self.block_max = torch.empty((Q, _round_up(max(nbm, 1), 64)), dtype=f32, device=device)
        self.pool_scores = torch.empty((Q, _round_up(self.pool_cols, 64)), dtype=f32, device=device)
        self.cand = torch.empty((Q, wl.n_blocks), dtype=torch.int32, device=device)
        # A pool-building Full layer may skip writing its scores: the block
        # maxima rank its best blocks, whose keys are scored again (pool
        # mode, the same arithmetic, so the same values) and selected from.
        # Worth it where the score writes cost more than the extra launches:
        # decode batches (the query-tiled prefill scorer stages its writes)
        # with many keys per call.
        if rescore is None:
            rescore = (self.quant and Q < RESCORE_MAX_Q and Q * self.n_cols >= RESCORE_MIN_KEYS)
        self.rescore = bool(rescore) and self.quant and self.fuse_block_max and wl.topk <= 4096
        # In the overlapped schedule (steps(concurrent=True)) a pool-building
        # Full layer whose attention runs on the second stream finishes its
        # top-k on that stream too, so the main stream needs only the pool
        # before the next layer's scoring: on this route the re-scoring and
        # its top-k, else the top-k through the block maxima
        # (side_topk_blocks), beside the pool's own ranking on the main
        # stream.
        self.side_topk_blocks = self.via_blocks and not self.rescore
        self.top_cols = wl.topk * wl.block_size
        # best blocks and their re-scored keys, per pool-building Full layer
        # (a layer finishing on the second stream may still read its own
        # while a later one ranks blocks on the main stream)
        self.top_bufs = {}
        if self.rescore:
            for li, l in enumerate(wl.layers):
                if l.mode == "full" and self.needs_pool[li]:
                    self.top_bufs[li] = (
                        torch.empty((Q, wl.topk), dtype=torch.int32, device=device),
                        torch.empty((Q, _round_up(self.top_cols, 64)), dtype=f32, device=device))
        first = self.top_bufs[min(self.top_bufs)] if self.top_bufs else (None, None)
        self.top_blocks, self.top_scores = first
        self.idx = {li: torch.empty((Q, wl.topk), dtype=torch.int32, device=device)
                    for li, l in enumerate(wl.layers) if l.mode in ("full", "reindex")}
        ws = max(csa2_topk_workspace_size(Q, self.n_cols, wl.topk),
                 csa2_topk_workspace_size(Q, self.pool_cols, wl.topk),
                 csa2_block_candidates_workspace_size(Q, self.n_cols, wl.block_size, wl.n_blocks),
                 csa2_topk_and_block_candidates_workspace_size(Q, self.n_cols, wl.topk,
                                                               wl.block_size, wl.n_blocks),
                 csa2_topk_from_block_max_workspace_size(Q, self.n_cols, wl.topk, wl.block_size),
                 csa2_top_blocks_and_block_candidates_workspace_size(Q, self.n_cols, wl.block_size, wl.topk,
                                                                     wl.n_blocks) if self.top_bufs else 0,
                 csa2_topk_workspace_size(Q, self.top_cols, wl.topk) if self.top_bufs else 0)
        self.ws = torch.empty((max(ws, 16),), dtype=torch.uint8, device=device)
        # a Full layer's top-k when it runs on the second stream, beside the
        # main stream's selections
        ws_t = max(csa2_topk_workspace_size(Q, self.top_cols, wl.topk) if self.top_bufs else 0,
                   csa2_topk_from_block_max_workspace_size(Q, self.n_cols, wl.topk, wl.block_size)
                   if self.side_topk_blocks else 0)
        self.ws_side = torch.empty((max(ws_t, 16),), dtype=torch.uint8, device=device)
        # block candidates may run beside the Full layer's top-k on a second
        # stream, so they get a workspace of their own
        ws_b = csa2_block_candidates_workspace_size(Q, self.n_cols, wl.block_size, wl.n_blocks)
        self.ws_blocks = torch.empty((max(ws_b, 16),), dtype=torch.uint8, device=device)
        self._side = None
        self._joined = None
        # attention splits keys over several workgroups at small batch sizes
        ws_a = csa2_sparse_attn_workspace_size(Q, 64, wl.topk, wl.window)
        self.ws_attn = (torch.empty((ws_a,), dtype=torch.uint8, device=device)
                        if ws_a > 0 else None)
        odt = torch.bfloat16 if self.quant else f32
        self.out = [torch.empty((Q, 64, 512), dtype=odt, device=device) for _ in wl.layers]
        self.lse = [torch.empty((Q, 64), dtype=f32, device=device) for _ in wl.layers]
        self.pages_scores = self.pages_topk = None
        self.n_main_rows = 0
        if paged is not None:
            pl = paged
            base = pl.k_pool.data_ptr()
            fp4 = getattr(wl, "k_fmt", "fp8") == "fp4s16"
            self.k_rows = csa2_rows(base, base + pl.k_scale_offset, pl.k_row_bytes,
                                    8 if fp4 else 1,
                                    CSA2_FP4_E2M1_E4M3S16 if fp4 else CSA2_FP8_E4M3)
            self.main_rows = (rows_fp4s16_records(pl.main_pool) if pl.main_pool.shape[1] == 288
                              else rows_fp4_records(pl.main_pool))
            self.n_main_rows = pl.main_pool.shape[0]
            self.pages_scores = csa2_pages(pl.page_table.data_ptr(), pl.page_table.shape[1],
                                           pl.n_pages, pl.k_page_bytes, None)
            self.pages_topk = csa2_pages(pl.page_table.data_ptr(), pl.page_table.shape[1],
                                         pl.n_pages, 0, wl.q_seq.data_ptr())
        self.slots = SlotSet(self.main_rows, self.k_rows)

    # -- steps -----------------------------------------------------------------
    def index_scores(self, li, pool, block_max=False, scores=True):
        wl, lay = self.wl, self.wl.layers[li]
        wdt = CSA2_BF16 if self.quant else CSA2_F32
        if pool == "top":
            # the keys of the Full layer's best blocks, scored again
            top_blocks, top_scores = self.top_bufs[li]
            csa2_index_scores(self.layer_rows[li]["q_idx"], lay.w, wdt, self.slots.index_k,
                              wl.seq_base, wl.q_seq, wl.q_pos, wl.ratio, top_scores,
                              self.top_cols, self.Q, cand=top_blocks,
                              block_size=wl.block_size, pages=self.pages_scores)
        elif pool:
            csa2_index_scores(self.layer_rows[li]["q_idx"], lay.w, wdt, self.slots.index_k,
                              wl.seq_base, wl.q_seq, wl.q_pos, wl.ratio, self.pool_scores,
                              self.pool_cols, self.Q, cand=self.slots.candidates,
                              block_size=wl.block_size, pages=self.pages_scores)
        else:
            csa2_index_scores(self.layer_rows[li]["q_idx"], lay.w, wdt, self.slots.index_k,
                              wl.seq_base, wl.q_seq, wl.q_pos, wl.ratio,
                              self.scores if scores else None,
                              self.n_cols, self.Q, block_size=wl.block_size,
                              block_max=self.block_max if block_max else None,
                              pages=self.pages_scores)

    def block_candidates(self, from_block_max=False):
        wl = self.wl
        csa2_block_candidates(self.scores, self.n_cols, wl.q_pos, wl.ratio, wl.block_size,
                              wl.n_blocks, self.cand, self.ws_blocks, self.Q,
                              block_max=self.block_max if from_block_max else None)
        self.slots.candidates = self.cand

    def topk(self, li, pool, via_blocks=False, ws=None):
        wl = self.wl
        idx = self.idx[li]
        if via_blocks:
            csa2_topk_from_block_max(self.scores, self.n_cols, self.block_max, wl.q_pos, wl.ratio,
                                     wl.block_size, wl.topk, idx, self.ws if ws is None else ws, self.Q,
                                     pages=self.pages_topk)
        elif pool:
            csa2_topk(self.pool_scores, self.pool_cols, None, wl.ratio, wl.topk, idx, self.ws,
                      self.Q, cand=self.slots.candidates, block_size=wl.block_size,
                      pages=self.pages_topk)
        else:
            csa2_topk(self.scores, self.n_cols, wl.q_pos, wl.ratio, wl.topk, idx, self.ws, self.Q,
                      pages=self.pages_topk)
        self.slots.topk_idxs = idx

    def top_blocks_and_blocks(self, li):
        """Full layer li's best blocks and the candidate pool, from its block
        maxima (no scores written)."""
        wl = self.wl
        csa2_top_blocks_and_block_candidates(self.block_max, self.n_cols, wl.q_pos, wl.ratio,
                                             wl.block_size, wl.topk, self.top_bufs[li][0], wl.n_blocks,
                                             self.cand, self.ws, self.Q)
        self.slots.candidates = self.cand

    def topk_top(self, li, ws=None):
        """Full layer li's top-k among its best blocks' re-scored keys."""
        wl = self.wl
        idx = self.idx[li]
        top_blocks, top_scores = self.top_bufs[li]
        csa2_topk(top_scores, self.top_cols, None, wl.ratio, wl.topk, idx,
                  self.ws if ws is None else ws, self.Q,
                  cand=top_blocks, block_size=wl.block_size, pages=self.pages_topk)
        self.slots.topk_idxs = idx

    def topk_and_blocks(self, li, from_block_max=False):
        """The Full layer's top-k and the candidate pool in shared launches."""
        wl = self.wl
        idx = self.idx[li]
        csa2_topk_and_block_candidates(self.scores, self.n_cols, wl.q_pos, wl.ratio, wl.topk, idx,
                                       wl.block_size, wl.n_blocks, self.cand, self.ws, self.Q,
                                       block_max=self.block_max if from_block_max else None,
                                       pages=self.pages_topk)
        self.slots.topk_idxs = idx
        self.slots.candidates = self.cand

    def attention(self, li):
        wl, lay = self.wl, self.wl.layers[li]
        qdt = CSA2_BF16 if self.quant else CSA2_F32
        csa2_sparse_attn(lay.q, qdt, self.slots.compress_kv, wl.seq_base, self.slots.topk_idxs,
                         wl.topk, self.layer_rows[li]["swa"], wl.swa_base, wl.swa_pos0, None,
                         wl.window, wl.q_seq, wl.q_pos, wl.ratio, lay.sink, wl.softmax_scale,
                         self.out[li], qdt if self.quant else CSA2_F32, self.lse[li], self.Q,
                         workspace=self.ws_attn, rope_cs=self.rope_cs,
                         idx_slots=self.paged is not None, n_main_rows=self.n_main_rows)

    # -- a whole pass ----------------------------------------------------------
    def fuses_block_max(self, li):
        """Whether layer li's dense scoring pass also writes block maxima."""
        return self.fuse_block_max and (self.needs_pool[li] or self.via_blocks)

    def rescored(self, li, overlap_route=False):
        """Whether Full layer li takes the re-scoring route (writes only its
        block maxima)."""
        return self.wl.layers[li].mode == "full" and self.needs_pool[li] and self.rescore

    def steps(self, concurrent=False, separate_select=False, overlap_route=None):
        """The calls of one pass over every layer, in order, as (stage name,
        callable) pairs.

        With rescore, a pool-building Full layer writes only its block
        maxima; csa2_top_blocks_and_block_candidates ranks its best blocks and
        the pool, and its top-k is taken among the best blocks' keys scored
        again (the same values, so the same top-k).  Otherwise a Full layer's
        dense scoring writes the block maxima when its top-k
        ranks blocks first (via_blocks) or a later layer needs the pool; the
        selections then read those maxima.  A Full layer that builds the pool
        makes both of its selections with one call
        (csa2_topk_and_block_candidates) unless separate_select asks for two
        calls; a Full layer's own top-k alone is csa2_topk_from_block_max
        (via_blocks) or csa2_topk.

        concurrent=True issues the attention calls that a later layer's
        scoring and selection can overlap on a second stream, in layer
        order: such a call waits only for the work issued before it on the
        main stream (its own top-k); the attention calls after the last
        scoring layer run on the main stream once the second stream's work
        is done (nothing is left to overlap them).  A pool-building Full
        layer whose attention goes to the second stream finishes its top-k
        on that stream before the attention (the re-scoring and its top-k,
        or the top-k through the block maxima with the pool ranked
        separately on the main stream), so the next layers need only the
        pool; overlap_route=True (the default with concurrent) takes the
        same route with every call on one stream.
        Attention calls stay in
        order among themselves (they share the split workspace), and every
        buffer an attention call reads is written before it (on the main
        stream, or ahead of it on the second) and not again within the pass (each layer has its own top-k
        buffer).  Each callable launches on the stream current when it is
        called, so the pass can be captured into one graph."""
        out = []

        def reset():
            self.slots.topk_idxs = None
            self.slots.candidates = None
        out.append(("reset", reset))
        has_pool = False
        layers = self.wl.layers
        last_scoring = max((i for i, l in enumerate(layers) if l.mode in ("full", "reindex")), default=-1)
        joined = False
        if overlap_route is None:
            overlap_route = concurrent
        for li, lay in enumerate(layers):
            side = concurrent and li < last_scoring
            if not separate_select and self.rescored(li):
                out.append(("index_scores_dense",
                            lambda li=li: self.index_scores(li, pool=False, block_max=True, scores=False)))
                out.append(("top_blocks_and_blocks", lambda li=li: self.top_blocks_and_blocks(li)))
                has_pool = True
                if side:
                    # re-scoring, top-k and attention on the second stream
                    out.append(("topk_top_and_sparse_attn", lambda li=li: self._attention_side(
                        li, before=(lambda: self.index_scores(li, pool="top"),
                                    lambda: self.topk_top(li, ws=self.ws_side)))))
                    continue
                out.append(("index_scores_top", lambda li=li: self.index_scores(li, pool="top")))
                out.append(("topk_top", lambda li=li: self.topk_top(li)))
            elif (lay.mode == "full" and self.needs_pool[li] and not separate_select and overlap_route
                  and self.side_topk_blocks and not any(l.mode == "full" for l in layers[li + 1:])):
                # the pool's ranking on the main stream, the top-k through
                # the block maxima beside it (it reads the layer's scores and
                # maxima, so no later Full layer may rewrite them meanwhile)
                out.append(("index_scores_dense",
                            lambda li=li: self.index_scores(li, pool=False, block_max=True)))
                has_pool = True
                if side:
                    out.append(("topk_blocks_and_sparse_attn", lambda li=li: self._attention_side(
                        li, before=(lambda: self.topk(li, pool=False, via_blocks=True, ws=self.ws_side),))))
                    out.append(("block_candidates", lambda: self.block_candidates(from_block_max=True)))
                    continue
                out.append(("topk_blocks", lambda li=li: self.topk(li, pool=False, via_blocks=True)))
                out.append(("block_candidates", lambda: self.block_candidates(from_block_max=True)))
            elif lay.mode == "full":
                fuse = self.fuses_block_max(li)
                out.append(("index_scores_dense",
                            lambda li=li, fuse=fuse: self.index_scores(li, pool=False, block_max=fuse)))
                if self.needs_pool[li] and not separate_select:
                    out.append(("topk_and_blocks",
                                lambda li=li, fuse=fuse: self.topk_and_blocks(li, fuse)))
                    has_pool = True
                else:
                    if self.needs_pool[li]:
                        out.append(("block_candidates",
                                    lambda fuse=fuse: self.block_candidates(from_block_max=fuse)))
                        has_pool = True
                    if self.via_blocks:
                        out.append(("topk_blocks", lambda li=li: self.topk(li, pool=False, via_blocks=True)))
                    else:
                        out.append(("topk_dense", lambda li=li: self.topk(li, pool=False)))
            elif lay.mode == "reindex":
                pool = has_pool
                out.append(("index_scores_pool" if pool else "index_scores_dense",
                            lambda li=li, pool=pool: self.index_scores(li, pool=pool)))
                out.append(("topk_pool" if pool else "topk_dense",
                            lambda li=li, pool=pool: self.topk(li, pool=pool)))
            if side:
                out.append(("sparse_attn", lambda li=li: self._attention_side(li)))
            else:
                if concurrent and not joined:
                    out.append(("join", self._join))
                    joined = True
                out.append(("sparse_attn", lambda li=li: self.attention(li)))
        if concurrent and not joined:
            out.append(("join", self._join))
        return out

    def _attention_side(self, li, before=()):
        """Layer li's attention (after the callables in before) on the second
        stream, after everything issued so far on the current stream."""
        main = torch.cuda.current_stream()
        if self._side is None:
            self._side = torch.cuda.Stream(device=main.device)   # default priority
        ready = torch.cuda.Event()
        ready.record(main)
        self._side.wait_event(ready)
        with torch.cuda.stream(self._side):
            for fn in before:
                fn()
            self.attention(li)
        self._joined = torch.cuda.Event()
        self._joined.record(self._side)

    def _join(self):
        if self._joined is not None:
            torch.cuda.current_stream().wait_event(self._joined)
            self._joined = None

    def run(self, mark=None, concurrent=False, separate_select=False):
        """Run every layer once.  mark(name) is called before each step and
        once at the end with None (the benchmark records events there)."""
        for name, fn in self.steps(concurrent, separate_select):
            if name not in ("reset", "join") and mark:
                mark(name)
            fn()
        if mark:
            mark(None)
        return self.out
