"""Turn a synthetic workload's byte tensors into the oracle's float64 inputs.

Only the oracle's own decoders are used here.
"""
import numpy as np

import oracle


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def index_q(layer, quantized):
    if quantized:
        return oracle.decode_e4m3_rows(_np(layer.q_idx), _np(layer.q_scale))
    return _np(layer.q_idx).astype(np.float64)


def index_w(layer, quantized):
    if quantized:
        return oracle.decode_bf16(_np(layer.w))
    return _np(layer.w).astype(np.float64)


def index_k_rows(wl, rows=None):
    """Dequantized index keys (all rows, or the given row indices)."""
    k = wl.k_idx if rows is None else wl.k_idx[rows]
    if wl.quantized:
        s = wl.k_scale if rows is None else wl.k_scale[rows]
        if getattr(wl, "k_fmt", "fp8") == "fp4s16":
            return oracle.decode_fp4s16_rows(_np(k), _np(s))
        return oracle.decode_e4m3_rows(_np(k), _np(s))
    return _np(k).astype(np.float64)


def main_rows(wl, rows=None):
    m = wl.main_kv if rows is None else wl.main_kv[rows]
    if wl.quantized:
        if getattr(wl, "main_fmt", "fp4") == "fp4s16":
            return oracle.decode_fp4s16_records(_np(m))
        return oracle.decode_fp4_records(_np(m))
    return _np(m).astype(np.float64)


def attn_q(layer, quantized):
    if quantized:
        return oracle.decode_bf16(_np(layer.q))
    return _np(layer.q).astype(np.float64)


def swa_rows(layer, quantized):
    if quantized:
        return oracle.decode_swa_records(_np(layer.swa))
    return _np(layer.swa).astype(np.float64)


def meta(wl):
    return dict(seq_base=_np(wl.seq_base), q_seq=_np(wl.q_seq), q_pos=_np(wl.q_pos),
                swa_base=_np(wl.swa_base), swa_pos0=_np(wl.swa_pos0))


def oracle_layers(wl):
    out = []
    for lay in wl.layers:
        d = {"mode": lay.mode, "q": attn_q(lay, wl.quantized),
             "swa_rows": swa_rows(lay, wl.quantized), "sink": _np(lay.sink).astype(np.float64)}
        if lay.q_idx is not None:
            d["q_idx"] = index_q(lay, wl.quantized)
            d["w"] = index_w(lay, wl.quantized)
        out.append(d)
    return out


def run_oracle(wl, use_pool=True):
    m = meta(wl)
    return oracle.run_layers(oracle_layers(wl), index_k_rows(wl), main_rows(wl),
                             m["seq_base"], m["q_seq"], m["q_pos"], wl.ratio,
                             m["swa_base"], m["swa_pos0"], wl.window, wl.topk,
                             wl.block_size, wl.n_blocks, wl.softmax_scale,
                             use_pool=use_pool)
