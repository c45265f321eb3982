"""Python binding of libcsa2.so, the CSA2 global-attention hot path on MI355X.

The functions below carry the names of the C entry points and do only
argument marshalling: tensors become device pointers, the current torch
stream becomes the HIP stream, and a non-zero status raises Csa2Error.
Every step of the path runs in the library's HIP kernels; there is no
fallback.  PyTorch supplies device memory and streams.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

CSA2_OK, CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP = 0, -1, -2, -3, -4
CSA2_F32, CSA2_BF16, CSA2_FP8_E4M3, CSA2_FP4_E2M1, CSA2_FP4_E2M1_E4M3S16 = 0, 1, 2, 3, 4

EXPORTED = ("csa2_index_scores", "csa2_block_candidates", "csa2_block_candidates_workspace_size",
            "csa2_topk", "csa2_topk_workspace_size", "csa2_topk_and_block_candidates",
            "csa2_topk_and_block_candidates_workspace_size",
            "csa2_topk_and_block_candidates_noalloc", "csa2_noalloc_scratch_bytes",
            "csa2_diag_index_scores_fp8_mfma", "csa2_diag_stream_read", "csa2_diag_stream_write",
            "csa2_diag_mfma_valu", "csa2_top_blocks_and_block_candidates",
            "csa2_top_blocks_and_block_candidates_workspace_size",
            "csa2_topk_from_block_max", "csa2_topk_from_block_max_workspace_size", "csa2_sparse_attn",
            "csa2_sparse_attn_workspace_size", "csa2_cache_write",
            "csa2_status_string", "csa2_last_error", "csa2_version")


class Csa2Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class csa2_pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
                ("n_pages", ctypes.c_int32), ("page_stride", ctypes.c_int64),
                ("q_seq", ctypes.c_void_p)]


def pages_of(table, n_pages=0, page_stride=0, q_seq=None):
    """csa2_pages over an int32 [B, n] page table tensor."""
    assert table.dtype == torch.int32 and table.is_contiguous() and table.dim() == 2
    return csa2_pages(table.data_ptr(), table.shape[1], n_pages, page_stride,
                      None if q_seq is None else q_seq.data_ptr())


class csa2_attn_io(ctypes.Structure):
    _fields_ = [("rope_cs", ctypes.c_void_p), ("n_rope", ctypes.c_int32),
                ("idx_slots", ctypes.c_int32), ("n_main_rows", ctypes.c_int64)]


class csa2_rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("row_stride", ctypes.c_int64), ("scale_stride", ctypes.c_int64),
                ("dtype", ctypes.c_int)]


_lib = None


def load():
    """Load libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing; run `python -m top_sparse_long_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    RP = ctypes.POINTER(csa2_rows)
    PP = ctypes.POINTER(csa2_pages)
    lib.csa2_index_scores.argtypes = [RP, P, ctypes.c_int, RP, P, P, P, I32, P, I32, I32, P, I64,
                                      I32, P, I64, I32, I32, I32, PP, P]
    lib.csa2_block_candidates.argtypes = [P, I64, I32, P, I64, P, I32, I32, I32, P, P, SZ, I32, P]
    lib.csa2_block_candidates_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.csa2_block_candidates_workspace_size.restype = SZ
    lib.csa2_topk.argtypes = [P, I64, I32, P, I32, P, I32, I32, I32, P, P, SZ, I32, PP, P]
    lib.csa2_topk_workspace_size.argtypes = [I32, I32, I32]
    lib.csa2_topk_workspace_size.restype = SZ
    lib.csa2_topk_and_block_candidates.argtypes = [P, I64, I32, P, I64, P, I32, I32, P, I32, I32,
                                                   P, P, SZ, I32, PP, P]
    lib.csa2_topk_and_block_candidates_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.csa2_topk_and_block_candidates_workspace_size.restype = SZ
    lib.csa2_topk_and_block_candidates_noalloc.argtypes = [P, I64, I32, P, I64, P, I32, I32, P, I32,
                                                           I32, P, I32, PP, P]
    lib.csa2_diag_stream_read.argtypes = [P, SZ, P, SZ, P]
    lib.csa2_diag_stream_write.argtypes = [P, SZ, ctypes.c_float, P]
    lib.csa2_diag_mfma_valu.argtypes = [I32, I32, P, SZ, P]
    lib.csa2_top_blocks_and_block_candidates.argtypes = [P, I64, I32, P, I32, I32, I32, P, I32, P, P, SZ,
                                                         I32, P]
    lib.csa2_top_blocks_and_block_candidates_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.csa2_top_blocks_and_block_candidates_workspace_size.restype = SZ
    lib.csa2_topk_from_block_max.argtypes = [P, I64, I32, P, I64, P, I32, I32, I32, P, P, SZ, I32, PP, P]
    lib.csa2_topk_from_block_max_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.csa2_topk_from_block_max_workspace_size.restype = SZ
    lib.csa2_diag_index_scores_fp8_mfma.argtypes = [RP, P, ctypes.c_int, RP, P, P, P, I32, P, I64, I32,
                                                    I32, P]
    lib.csa2_noalloc_scratch_bytes.argtypes = []
    lib.csa2_noalloc_scratch_bytes.restype = SZ
    lib.csa2_sparse_attn.argtypes = [P, ctypes.c_int, RP, P, P, I32, RP, P, P, P, I32, P, P, I32,
                                     P, ctypes.c_float, P, ctypes.c_int, P, P, SZ, I32, I32, I32,
                                     ctypes.POINTER(csa2_attn_io), P]
    lib.csa2_sparse_attn_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.csa2_sparse_attn_workspace_size.restype = SZ
    lib.csa2_cache_write.argtypes = [P, P, I64, P, P, I32, I32, P, I32, P, P, P, ctypes.c_float,
                                     P, I32, RP, P, I64, RP, P, I64, P]
    lib.csa2_status_string.argtypes = [ctypes.c_int]
    lib.csa2_status_string.restype = ctypes.c_char_p
    lib.csa2_last_error.restype = ctypes.c_char_p
    for fn in ("csa2_index_scores", "csa2_block_candidates", "csa2_topk",
               "csa2_topk_and_block_candidates", "csa2_topk_and_block_candidates_noalloc",
               "csa2_diag_index_scores_fp8_mfma", "csa2_diag_stream_read", "csa2_diag_stream_write",
               "csa2_diag_mfma_valu", "csa2_topk_from_block_max", "csa2_sparse_attn", "csa2_cache_write",
               "csa2_top_blocks_and_block_candidates",
               "csa2_version"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != CSA2_OK:
        lib = load()
        raise Csa2Error(status, lib.csa2_last_error().decode() or
                        lib.csa2_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# row descriptors

def rows_f32(x):
    """fp32 [n, dim] rows."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    return csa2_rows(x.data_ptr(), None, x.shape[-1] * 4, 0, CSA2_F32)


def rows_fp8(codes, scale):
    """E4M3 codes [n, dim] (uint8) with one fp32 scale per row [n]."""
    assert codes.dtype == torch.uint8 and codes.is_contiguous() and scale.dtype == torch.float32
    return csa2_rows(codes.data_ptr(), scale.data_ptr(), codes.shape[-1],
                     scale.stride(0) if scale.dim() else 1, CSA2_FP8_E4M3)


def rows_fp4s16(codes, scales):
    """E2M1 codes [n, dim / 2] (uint8, two per byte) with one E4M3 scale byte
    per 16 elements [n, dim / 16] (uint8): the pages' FP4 cache format."""
    assert codes.dtype == torch.uint8 and codes.is_contiguous()
    assert scales.dtype == torch.uint8 and scales.dim() == 2
    return csa2_rows(codes.data_ptr(), scales.data_ptr(), codes.shape[-1], scales.stride(0),
                     CSA2_FP4_E2M1_E4M3S16)


def rows_fp4_records(rec):
    """320-byte FP4 main-KV records [n, 320]: 256 code bytes, 16 fp32 scales."""
    assert rec.dtype == torch.uint8 and rec.is_contiguous() and rec.shape[-1] == 320
    return csa2_rows(rec.data_ptr(), rec.data_ptr() + 256, 320, 80, CSA2_FP4_E2M1)


def rows_fp4s16_records(rec):
    """The pages' 288-byte main-KV records [n, 288]: 256 code bytes, then 32
    E4M3 scale bytes (one per 16 elements)."""
    assert rec.dtype == torch.uint8 and rec.is_contiguous() and rec.shape[-1] == 288
    return csa2_rows(rec.data_ptr(), rec.data_ptr() + 256, 288, 288, CSA2_FP4_E2M1_E4M3S16)


def rows_swa_records(rec):
    """528-byte FP8 SWA records [n, 528]: 512 code bytes, 4 fp32 scales."""
    assert rec.dtype == torch.uint8 and rec.is_contiguous() and rec.shape[-1] == 528
    return csa2_rows(rec.data_ptr(), rec.data_ptr() + 512, 528, 132, CSA2_FP8_E4M3)


# ---------------------------------------------------------------------------
# the calls

def _byref(x):
    return None if x is None else ctypes.byref(x)


def csa2_index_scores(q_rows, w, w_dtype, k_rows, seq_base, q_seq, q_pos, ratio, scores,
                      n_cols, Q, cand=None, block_size=8, block_max=None, H_I=32, d_I=128,
                      stream=None, pages=None):
    """pages: an optional csa2_pages (paged index-key cache)."""
    lib = load()
    ncb = 0 if cand is None else cand.shape[-1]
    bms = 0 if block_max is None else block_max.stride(0)
    _check(lib.csa2_index_scores(ctypes.byref(q_rows), _ptr(w), w_dtype, ctypes.byref(k_rows),
                                 _ptr(seq_base), _ptr(q_seq), _ptr(q_pos), ratio, _ptr(cand), ncb,
                                 block_size, _ptr(scores), 0 if scores is None else scores.stride(0), n_cols,
                                 _ptr(block_max), bms, Q, H_I, d_I, _byref(pages),
                                 _stream(stream)))


def csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks):
    return load().csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks)


def csa2_topk_workspace_size(Q, n_cols, k):
    return load().csa2_topk_workspace_size(Q, n_cols, k)


def csa2_block_candidates(scores, n_cols, q_pos, ratio, block_size, n_blocks, cand, workspace,
                          Q, block_max=None, stream=None):
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sst = 0 if scores is None else scores.stride(0)
    bms = 0 if block_max is None else block_max.stride(0)
    _check(lib.csa2_block_candidates(_ptr(scores), sst, n_cols, _ptr(block_max), bms,
                                     _ptr(q_pos), ratio, block_size, n_blocks, _ptr(cand),
                                     _ptr(workspace), wsb, Q, _stream(stream)))


def csa2_topk(scores, n_cols, q_pos, ratio, k, idx, workspace, Q, cand=None, block_size=8,
              stream=None, pages=None):
    """pages: an optional csa2_pages (table, q_seq): idx receives slots."""
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ncb = 0 if cand is None else cand.shape[-1]
    _check(lib.csa2_topk(_ptr(scores), scores.stride(0), n_cols, _ptr(q_pos), ratio, _ptr(cand),
                         ncb, block_size, k, _ptr(idx), _ptr(workspace), wsb, Q, _byref(pages),
                         _stream(stream)))


def csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, block_size, n_blocks):
    return load().csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, block_size,
                                                                n_blocks)


def csa2_diag_index_scores_fp8_mfma(q_rows, w, w_dtype, k_rows, seq_base, q_seq, q_pos, ratio,
                                    scores, n_cols, Q, stream=None):
    """Diagnostic: dense FP8 scores with the dot products on the FP8 matrix cores."""
    _check(load().csa2_diag_index_scores_fp8_mfma(ctypes.byref(q_rows), _ptr(w), w_dtype,
                                                  ctypes.byref(k_rows), _ptr(seq_base), _ptr(q_seq),
                                                  _ptr(q_pos), ratio, _ptr(scores), scores.stride(0),
                                                  n_cols, Q, _stream(stream)))


def csa2_diag_stream_read(src, sink, stream=None):
    """Diagnostic: read the whole of src (a device tensor) once at full speed."""
    _check(load().csa2_diag_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                        sink.numel(), _stream(stream)))


def csa2_diag_stream_write(dst, value=0.0, stream=None):
    """Diagnostic: fill the whole of dst (a device tensor) at full speed."""
    _check(load().csa2_diag_stream_write(_ptr(dst), dst.numel() * dst.element_size(), value,
                                         _stream(stream)))


def csa2_diag_mfma_valu(mode, iters, sink, stream=None):
    """Diagnostic: the MFMA / VALU overlap loop (mode 1 products, 2 FMAs,
    3 both) into sink, a device float tensor of at least 256 * 512 values."""
    _check(load().csa2_diag_mfma_valu(mode, iters, _ptr(sink), sink.numel(), _stream(stream)))


def csa2_topk_from_block_max_workspace_size(Q, n_cols, k, block_size):
    return load().csa2_topk_from_block_max_workspace_size(Q, n_cols, k, block_size)


def csa2_topk_from_block_max(scores, n_cols, block_max, q_pos, ratio, block_size, k, idx, workspace,
                             Q, stream=None, pages=None):
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.csa2_topk_from_block_max(_ptr(scores), scores.stride(0), n_cols, _ptr(block_max),
                                        block_max.stride(0), _ptr(q_pos), ratio, block_size, k,
                                        _ptr(idx), _ptr(workspace), wsb, Q, _byref(pages),
                                        _stream(stream)))


def csa2_noalloc_scratch_bytes():
    return load().csa2_noalloc_scratch_bytes()


def csa2_topk_and_block_candidates_noalloc(scores, n_cols, q_pos, ratio, k, idx, block_size,
                                           n_blocks, cand, Q, block_max=None, stream=None,
                                           pages=None):
    lib = load()
    bms = 0 if block_max is None else block_max.stride(0)
    _check(lib.csa2_topk_and_block_candidates_noalloc(_ptr(scores), scores.stride(0), n_cols,
                                                      _ptr(block_max), bms, _ptr(q_pos), ratio, k,
                                                      _ptr(idx), block_size, n_blocks, _ptr(cand), Q,
                                                      _byref(pages), _stream(stream)))


def csa2_topk_and_block_candidates(scores, n_cols, q_pos, ratio, k, idx, block_size, n_blocks,
                                   cand, workspace, Q, block_max=None, stream=None, pages=None):
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bms = 0 if block_max is None else block_max.stride(0)
    _check(lib.csa2_topk_and_block_candidates(_ptr(scores), scores.stride(0), n_cols,
                                              _ptr(block_max), bms, _ptr(q_pos), ratio, k,
                                              _ptr(idx), block_size, n_blocks, _ptr(cand),
                                              _ptr(workspace), wsb, Q, _byref(pages),
                                              _stream(stream)))


def csa2_top_blocks_and_block_candidates_workspace_size(Q, n_cols, block_size, k_blocks, n_blocks):
    return load().csa2_top_blocks_and_block_candidates_workspace_size(Q, n_cols, block_size, k_blocks,
                                                                      n_blocks)


def csa2_top_blocks_and_block_candidates(block_max, n_cols, q_pos, ratio, block_size, k_blocks,
                                         top_blocks, n_blocks, cand, workspace, Q, stream=None):
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.csa2_top_blocks_and_block_candidates(_ptr(block_max), block_max.stride(0), n_cols,
                                                    _ptr(q_pos), ratio, block_size, k_blocks,
                                                    _ptr(top_blocks), n_blocks, _ptr(cand),
                                                    _ptr(workspace), wsb, Q, _stream(stream)))


def csa2_sparse_attn_workspace_size(Q, H, k, window):
    return load().csa2_sparse_attn_workspace_size(Q, H, k, window)


def csa2_sparse_attn(q, q_dtype, main_rows, main_base, idx, k, swa_rows, swa_base, swa_pos0,
                     swa_lo, window, q_seq, q_pos, ratio, attn_sink, softmax_scale, out,
                     out_dtype, lse, Q, H=64, D=512, stream=None, workspace=None, rope_cs=None,
                     idx_slots=False, n_main_rows=0):
    """rope_cs: optional [n, 64] fp32 table (the output is turned back by
    each query's position); idx_slots: idx holds physical main rows."""
    lib = load()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    io = None
    if rope_cs is not None or idx_slots:
        io = csa2_attn_io(None if rope_cs is None else rope_cs.data_ptr(),
                          0 if rope_cs is None else rope_cs.shape[0], int(bool(idx_slots)),
                          n_main_rows)
    _check(lib.csa2_sparse_attn(_ptr(q), q_dtype, ctypes.byref(main_rows), _ptr(main_base),
                                _ptr(idx), k, ctypes.byref(swa_rows), _ptr(swa_base),
                                _ptr(swa_pos0), _ptr(swa_lo), window, _ptr(q_seq), _ptr(q_pos),
                                ratio, _ptr(attn_sink), ctypes.c_float(softmax_scale), _ptr(out),
                                out_dtype, _ptr(lse), _ptr(workspace), wsb, Q, H, D,
                                None if io is None else ctypes.byref(io), _stream(stream)))


def csa2_cache_write(c, z, tok_seq, tok_pos, ratio, pend, n_seq, kv_norm_w, w_ik, k_norm_w,
                     eps, rope_cs, main_rows, main_base, n_main_rows, k_rows, k_base,
                     n_k_rows, stream=None):
    """main_rows / k_rows: csa2_rows descriptors of the output rows, or None."""
    lib = load()
    T = 0 if tok_seq is None else tok_seq.numel()
    _check(lib.csa2_cache_write(_ptr(c), _ptr(z), c.stride(0) * c.element_size(), _ptr(tok_seq),
                                _ptr(tok_pos), T, ratio, _ptr(pend), n_seq, _ptr(kv_norm_w),
                                _ptr(w_ik), _ptr(k_norm_w), ctypes.c_float(eps), _ptr(rope_cs),
                                rope_cs.shape[0],
                                None if main_rows is None else ctypes.byref(main_rows),
                                _ptr(main_base), n_main_rows,
                                None if k_rows is None else ctypes.byref(k_rows),
                                _ptr(k_base), n_k_rows, _stream(stream)))
