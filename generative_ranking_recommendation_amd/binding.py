"""ctypes binding of libgenrank.so.  Argument marshalling only: each function builds the
C structs, passes device pointers and the current HIP stream, and raises GenrankError on a
non-zero status.  Every computation happens in the library's HIP kernels.

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed), plain integer
addresses, or None for optional pointers.  Host-array arguments (slopes, validate) take
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint8, c_uint32, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgenrank.so")

F32, BF16 = 0, 1
RESID_ACT, RESID_F32 = 0, 1
BLOCK_ATTN_ONLY, BLOCK_PRENORM = 0, 1
(OP_EMBED_SUM, OP_ATTN_FWD, OP_ATTN_BWD, OP_LAYER_FWD, OP_LAYER_BWD, OP_EMBED_BWD, OP_HEAD_BWD, OP_LAYER_KV,
 OP_LAYER_FWD_CACHED) = range(9)
FWD_SAVE = 1
EPI_NONE, EPI_RESIDUAL, EPI_SILU, EPI_RESIDUAL_F32 = 0, 1, 2, 3
STATUS = {0: "OK", -1: "E_ARG", -2: "E_SHAPE", -3: "E_DTYPE", -4: "E_UNSORTED",
          -5: "E_RANGE", -6: "E_WORKSPACE", -7: "E_HIP"}


class GenrankError(RuntimeError):
    def __init__(self, func, status):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} ({status})")


class Batch(Structure):
    _fields_ = [("B", c_int32), ("m", c_int32), ("d", c_int32), ("H", c_int32), ("dh", c_int32),
                ("max_hist", c_int32), ("total_hist", c_int64), ("dtype", c_int32),
                ("resid", c_int32)]


class Inputs(Structure):
    _fields_ = [("hist_offsets", c_void_p), ("hist_items", c_void_p), ("hist_actions", c_void_p),
                ("hist_ts", c_void_p), ("cand_items", c_void_p), ("req_ts", c_void_p)]


class Tables(Structure):
    _fields_ = [("item", c_void_p), ("action", c_void_p), ("pos", c_void_p), ("ri", c_void_p),
                ("rt", c_void_p), ("rt_bounds", c_void_p), ("n_item", c_int64),
                ("n_action", c_int32), ("n_pos", c_int32), ("n_ri", c_int32), ("n_rt", c_int32)]


class Alibi(Structure):
    _fields_ = [("slopes_pos", c_void_p), ("slopes_time", c_void_p), ("flags", c_int32),
                ("n_time_bounds", c_int32), ("time_bounds", c_void_p)]


ATTN_FULL_HISTORY = 1
ATTN_TIME_BUCKET = 2


class LayerWeights(Structure):
    _fields_ = [("wqkv", c_void_p), ("wo", c_void_p), ("w1", c_void_p), ("w2", c_void_p),
                ("g1", c_void_p), ("g2", c_void_p), ("ffn_dim", c_int32), ("block", c_int32),
                ("alibi", Alibi)]


class LayerGrads(Structure):
    _fields_ = [("wqkv", c_void_p), ("wo", c_void_p), ("w1", c_void_p), ("w2", c_void_p),
                ("g1", c_void_p), ("g2", c_void_p)]


# name -> (restype, argtypes)
_SIGS = {
    "genrank_status_string": (c_char_p, [c_int32]),
    "genrank_version": (c_int32, []),
    "genrank_workspace_size": (c_int32, [c_int32, POINTER(Batch), POINTER(LayerWeights), POINTER(c_size_t)]),
    "genrank_validate_host": (c_int32, [POINTER(Batch), POINTER(Inputs), POINTER(Tables), POINTER(c_int64)]),
    "genrank_error_word": (c_int32, [POINTER(c_uint32), c_int32, c_void_p]),
    "genrank_embed_sum": (c_int32, [POINTER(Batch), POINTER(Inputs), POINTER(Tables), c_void_p, c_void_p]),
    "genrank_attn_fwd": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, Alibi, c_void_p,
                                   c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p]),
    "genrank_attn_bwd": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, Alibi, c_void_p,
                                   c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                   c_void_p, c_size_t, c_void_p]),
    "genrank_attn_bwd_noalloc": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, Alibi, c_void_p,
                                           c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                           c_void_p]),
    "genrank_layer_fwd": (c_int32, [POINTER(Batch), POINTER(LayerWeights), c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                    c_void_p]),
    "genrank_layer_bwd": (c_int32, [POINTER(Batch), POINTER(LayerWeights), c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, LayerGrads,
                                    c_int32, c_void_p, c_size_t, c_void_p]),
    "genrank_linear": (c_int32, [c_int32, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                 c_int64, c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p,
                                 c_int64, c_void_p]),
    "genrank_linear_bwd_workspace": (c_int32, [c_int32, c_int64, c_int32, c_int32, POINTER(c_size_t)]),
    "genrank_linear_bwd": (c_int32, [c_int32, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                     c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int32, c_int32,
                                     c_void_p, c_size_t, c_void_p]),
    "genrank_embed_sum_cand": (c_int32, [POINTER(Batch), POINTER(Inputs), POINTER(Tables), c_void_p, c_void_p]),
    "genrank_attn_fwd_cached": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, Alibi, c_void_p, c_void_p,
                                          c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_void_p, c_int64,
                                          c_void_p, c_void_p]),
    "genrank_layer_kv": (c_int32, [POINTER(Batch), POINTER(LayerWeights), c_void_p, c_void_p, c_int64, c_void_p,
                                   c_size_t, c_void_p]),
    "genrank_layer_fwd_cached": (c_int32, [POINTER(Batch), POINTER(LayerWeights), c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "genrank_rmsnorm": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "genrank_head_fwd": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p]),
    "genrank_head_bwd": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
    "genrank_head_fwd_rows": (c_int32, [c_int32, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_void_p, c_void_p]),
    "genrank_head_bwd_rows": (c_int32, [c_int32, c_int32, c_int32, c_int64, c_void_p, c_int64, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_size_t, c_void_p]),
    "genrank_bce_loss": (c_int32, [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "genrank_embed_bwd": (c_int32, [POINTER(Batch), POINTER(Inputs), POINTER(Tables), c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "genrank_debug_indices": (c_int32, [POINTER(Batch), POINTER(Inputs), POINTER(Tables), c_void_p, c_void_p]),
    "genrank_debug_mask": (c_int32, [POINTER(Batch), c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "genrank_hstu_rab_layout": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p]),
    "genrank_hstu_rab": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "genrank_hstu_attn_fwd": (c_int32, [POINTER(Batch), c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                        c_void_p]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m generative_ranking_recommendation_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().genrank_status_string(int(status)).decode()


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name, status):
    if status != 0:
        raise GenrankError(name, status)


def make_batch(B, m, d, H, max_hist, total_hist, dtype, resid=RESID_ACT) -> Batch:
    return Batch(B=B, m=m, d=d, H=H, dh=d // H, max_hist=max_hist, total_hist=total_hist,
                 dtype=dtype, resid=resid)


def make_inputs(hist_offsets, hist_items, hist_actions, hist_ts, cand_items, req_ts) -> Inputs:
    return Inputs(_p(hist_offsets), _p(hist_items), _p(hist_actions), _p(hist_ts), _p(cand_items),
                  _p(req_ts))


def make_tables(item, action, pos, ri, rt, rt_bounds, n_item, n_action, n_pos, n_ri, n_rt) -> Tables:
    return Tables(_p(item), _p(action), _p(pos), _p(ri), _p(rt), _p(rt_bounds), n_item, n_action,
                  n_pos, n_ri, n_rt)


class HostSlopes:
    """Keeps the float32 host arrays alive for as long as the Alibi struct is used."""

    def __init__(self, slopes_pos, slopes_time, flags=0, time_bounds=None):
        """time_bounds: a device tensor of int64 edges (GENRANK_ATTN_TIME_BUCKET)."""
        self.sp = np.ascontiguousarray(slopes_pos, dtype=np.float32)
        self.st = np.ascontiguousarray(slopes_time, dtype=np.float32)
        self.time_bounds = time_bounds
        n = 0 if time_bounds is None else int(time_bounds.numel())
        self.struct = Alibi(self.sp.ctypes.data, self.st.ctypes.data, int(flags), n, _p(time_bounds))


def make_layer_weights(wqkv, wo, slopes: HostSlopes, block, w1=None, w2=None, g1=None, g2=None,
                       ffn_dim=0) -> LayerWeights:
    return LayerWeights(_p(wqkv), _p(wo), _p(w1), _p(w2), _p(g1), _p(g2), ffn_dim, block,
                        slopes.struct)


def make_layer_grads(wqkv, wo, w1=None, w2=None, g1=None, g2=None) -> LayerGrads:
    return LayerGrads(_p(wqkv), _p(wo), _p(w1), _p(w2), _p(g1), _p(g2))


# ---------------------------------------------------------------- entry points


def genrank_version() -> int:
    return lib().genrank_version()


def genrank_workspace_size(op, batch: Batch, weights: LayerWeights = None) -> int:
    n = c_size_t(0)
    _check("genrank_workspace_size", lib().genrank_workspace_size(
        op, ctypes.byref(batch), ctypes.byref(weights) if weights is not None else None, ctypes.byref(n)))
    return n.value


def genrank_validate_host(batch: Batch, inputs: Inputs, tables: Tables):
    """Returns (status, bad_row); does not raise (a non-zero status is the answer)."""
    bad = c_int64(-1)
    s = lib().genrank_validate_host(ctypes.byref(batch), ctypes.byref(inputs), ctypes.byref(tables),
                                    ctypes.byref(bad))
    return s, bad.value


ERR_ID_RANGE, ERR_HIST_LONG = 1, 2


def genrank_error_word(clear=True, stream=None) -> int:
    """The current device's error word (GENRANK_ERR_* bits), read after `stream` finishes;
    cleared afterwards unless clear is False."""
    w = c_uint32(0)
    _check("genrank_error_word", lib().genrank_error_word(ctypes.byref(w), int(bool(clear)), _stream(stream)))
    return int(w.value)


def genrank_embed_sum(batch, inputs, tables, x_out, stream=None):
    _check("genrank_embed_sum", lib().genrank_embed_sum(
        ctypes.byref(batch), ctypes.byref(inputs), ctypes.byref(tables), _p(x_out), _stream(stream)))


def genrank_attn_fwd(batch, hist_offsets, hist_ts, req_ts, slopes: HostSlopes, q, k, v, ld_qkv, o,
                     ld_o, lse=None, stream=None):
    _check("genrank_attn_fwd", lib().genrank_attn_fwd(
        ctypes.byref(batch), _p(hist_offsets), _p(hist_ts), _p(req_ts), slopes.struct, _p(q), _p(k),
        _p(v), ld_qkv, _p(o), ld_o, _p(lse), _stream(stream)))


def genrank_hstu_rab_layout(batch, hist_offsets, rab_offsets, stream=None):
    _check("genrank_hstu_rab_layout", lib().genrank_hstu_rab_layout(
        ctypes.byref(batch), _p(hist_offsets), _p(rab_offsets), _stream(stream)))


def genrank_hstu_rab(batch, hist_offsets, hist_ts, req_ts, pos_table, n_pos, time_table, time_bounds,
                     n_time, rab_offsets, rab, stream=None):
    _check("genrank_hstu_rab", lib().genrank_hstu_rab(
        ctypes.byref(batch), _p(hist_offsets), _p(hist_ts), _p(req_ts), _p(pos_table), n_pos,
        _p(time_table), _p(time_bounds), n_time, _p(rab_offsets), _p(rab), _stream(stream)))


def genrank_hstu_attn_fwd(batch, hist_offsets, rab, rab_offsets, q, k, v, ld_qkv, o, ld_o, lse=None,
                          stream=None):
    _check("genrank_hstu_attn_fwd", lib().genrank_hstu_attn_fwd(
        ctypes.byref(batch), _p(hist_offsets), _p(rab), _p(rab_offsets), _p(q), _p(k), _p(v), ld_qkv,
        _p(o), ld_o, _p(lse), _stream(stream)))


def genrank_attn_bwd(batch, hist_offsets, hist_ts, req_ts, slopes: HostSlopes, q, k, v, ld_qkv, o,
                     dout, ld_o, lse, dq, dk, dv, ld_dqkv, cand_only, ws, ws_bytes, stream=None):
    _check("genrank_attn_bwd", lib().genrank_attn_bwd(
        ctypes.byref(batch), _p(hist_offsets), _p(hist_ts), _p(req_ts), slopes.struct, _p(q), _p(k),
        _p(v), ld_qkv, _p(o), _p(dout), ld_o, _p(lse), _p(dq), _p(dk), _p(dv), ld_dqkv,
        int(cand_only), _p(ws), ws_bytes, _stream(stream)))


def genrank_attn_bwd_noalloc(batch, hist_offsets, hist_ts, req_ts, slopes: HostSlopes, q, k, v, ld_qkv, o,
                             dout, ld_o, lse, dq, dk, dv, ld_dqkv, cand_only, stream=None):
    _check("genrank_attn_bwd_noalloc", lib().genrank_attn_bwd_noalloc(
        ctypes.byref(batch), _p(hist_offsets), _p(hist_ts), _p(req_ts), slopes.struct, _p(q), _p(k),
        _p(v), ld_qkv, _p(o), _p(dout), ld_o, _p(lse), _p(dq), _p(dk), _p(dv), ld_dqkv,
        int(cand_only), _stream(stream)))


def genrank_layer_fwd(batch, weights: LayerWeights, hist_offsets, hist_ts, req_ts, x_in, y_out,
                      flags, ws, ws_bytes, stream=None):
    _check("genrank_layer_fwd", lib().genrank_layer_fwd(
        ctypes.byref(batch), ctypes.byref(weights), _p(hist_offsets), _p(hist_ts), _p(req_ts),
        _p(x_in), _p(y_out), flags, _p(ws), ws_bytes, _stream(stream)))


def genrank_layer_bwd(batch, weights: LayerWeights, hist_offsets, hist_ts, req_ts, x_in, ws, dy, dx,
                      grads: LayerGrads, cand_only, ws_bwd, ws_bwd_bytes, stream=None):
    _check("genrank_layer_bwd", lib().genrank_layer_bwd(
        ctypes.byref(batch), ctypes.byref(weights), _p(hist_offsets), _p(hist_ts), _p(req_ts),
        _p(x_in), _p(ws), _p(dy), _p(dx), grads, int(cand_only), _p(ws_bwd), ws_bwd_bytes,
        _stream(stream)))


def genrank_linear(dtype, x, ldx, w, ldw, y, ldy, M, N, K, epilogue=EPI_NONE, residual=None, ldr=0,
                   pre=None, ldpre=0, stream=None):
    _check("genrank_linear", lib().genrank_linear(
        dtype, _p(x), ldx, _p(w), ldw, _p(y), ldy, M, N, K, epilogue, _p(residual), ldr, _p(pre),
        ldpre, _stream(stream)))


def genrank_linear_bwd_workspace(dtype, M, N, K):
    n = c_size_t(0)
    _check("genrank_linear_bwd_workspace", lib().genrank_linear_bwd_workspace(dtype, M, N, K, ctypes.byref(n)))
    return n.value


def genrank_linear_bwd(dtype, x, ldx, w, ldw, dy, ldy, dx, lddx, dw, lddw, M, N, K, ws, ws_bytes,
                       stream=None):
    _check("genrank_linear_bwd", lib().genrank_linear_bwd(
        dtype, _p(x), ldx, _p(w), ldw, _p(dy), ldy, _p(dx), lddx, _p(dw), lddw, M, N, K, _p(ws),
        ws_bytes, _stream(stream)))


def genrank_embed_sum_cand(batch, inputs, tables, x_cand, stream=None):
    _check("genrank_embed_sum_cand", lib().genrank_embed_sum_cand(
        ctypes.byref(batch), ctypes.byref(inputs), ctypes.byref(tables), _p(x_cand), _stream(stream)))


def genrank_attn_fwd_cached(batch, hist_offsets, hist_ts, req_ts, slopes, q, k, v, ld_qkv, k_hist, v_hist,
                            ld_hist, o, ld_o, lse=None, stream=None):
    al = slopes.struct if isinstance(slopes, HostSlopes) else slopes
    _check("genrank_attn_fwd_cached", lib().genrank_attn_fwd_cached(
        ctypes.byref(batch), _p(hist_offsets), _p(hist_ts), _p(req_ts), al, _p(q), _p(k), _p(v), ld_qkv,
        _p(k_hist), _p(v_hist), ld_hist, _p(o), ld_o, _p(lse), _stream(stream)))


def genrank_layer_kv(batch, weights: LayerWeights, x_hist, kv, ld_kv, ws, ws_bytes, stream=None):
    _check("genrank_layer_kv", lib().genrank_layer_kv(
        ctypes.byref(batch), ctypes.byref(weights), _p(x_hist), _p(kv), ld_kv, _p(ws), ws_bytes,
        _stream(stream)))


def genrank_layer_fwd_cached(batch, weights: LayerWeights, hist_offsets, hist_ts, req_ts, kv_hist, ld_kv, x_cand,
                             y_cand, ws, ws_bytes, stream=None):
    _check("genrank_layer_fwd_cached", lib().genrank_layer_fwd_cached(
        ctypes.byref(batch), ctypes.byref(weights), _p(hist_offsets), _p(hist_ts), _p(req_ts), _p(kv_hist), ld_kv,
        _p(x_cand), _p(y_cand), _p(ws), ws_bytes, _stream(stream)))


def genrank_head_fwd(batch, x, g_final, w_head, b_head, n_tasks, logits, stream=None):
    _check("genrank_head_fwd", lib().genrank_head_fwd(
        ctypes.byref(batch), _p(x), _p(g_final), _p(w_head), _p(b_head), n_tasks, _p(logits),
        _stream(stream)))


def genrank_head_bwd(batch, x, g_final, w_head, n_tasks, dlogits, dx, dg_final, dw_head, db_head,
                     ws, ws_bytes, stream=None):
    _check("genrank_head_bwd", lib().genrank_head_bwd(
        ctypes.byref(batch), _p(x), _p(g_final), _p(w_head), n_tasks, _p(dlogits), _p(dx),
        _p(dg_final), _p(dw_head), _p(db_head), _p(ws), ws_bytes, _stream(stream)))


def genrank_rmsnorm(x_dtype, y_dtype, x, g, y, rows, d, stream=None):
    _check("genrank_rmsnorm", lib().genrank_rmsnorm(x_dtype, y_dtype, _p(x), _p(g), _p(y), rows, d,
                                                    _stream(stream)))


def genrank_head_fwd_rows(dtype, d, x, n_rows, rows, g_final, w_head, b_head, n_tasks, logits, stream=None):
    _check("genrank_head_fwd_rows", lib().genrank_head_fwd_rows(
        dtype, d, _p(x), n_rows, _p(rows), _p(g_final), _p(w_head), _p(b_head), n_tasks, _p(logits),
        _stream(stream)))


def genrank_head_bwd_rows(x_dtype, dtype, d, n_x_rows, x, n_rows, rows, g_final, w_head, n_tasks, dlogits, dx,
                          dg_final, dw_head, db_head, ws, ws_bytes, stream=None):
    _check("genrank_head_bwd_rows", lib().genrank_head_bwd_rows(
        x_dtype, dtype, d, n_x_rows, _p(x), n_rows, _p(rows), _p(g_final), _p(w_head), n_tasks, _p(dlogits), _p(dx),
        _p(dg_final), _p(dw_head), _p(db_head), _p(ws), ws_bytes, _stream(stream)))


def genrank_bce_loss(n, n_tasks, logits, labels, loss, dlogits, stream=None):
    _check("genrank_bce_loss", lib().genrank_bce_loss(
        n, n_tasks, _p(logits), _p(labels), _p(loss), _p(dlogits), _stream(stream)))


def genrank_embed_bwd(batch, inputs, tables, dx, item_ids, item_rows, n_items, d_action, d_pos, d_ri,
                      d_rt, ws, ws_bytes, stream=None):
    _check("genrank_embed_bwd", lib().genrank_embed_bwd(
        ctypes.byref(batch), ctypes.byref(inputs), ctypes.byref(tables), _p(dx), _p(item_ids),
        _p(item_rows), _p(n_items), _p(d_action), _p(d_pos), _p(d_ri), _p(d_rt), _p(ws), ws_bytes,
        _stream(stream)))


def genrank_debug_indices(batch, inputs, tables, out, stream=None):
    _check("genrank_debug_indices", lib().genrank_debug_indices(
        ctypes.byref(batch), ctypes.byref(inputs), ctypes.byref(tables), _p(out), _stream(stream)))


def genrank_debug_mask(batch, hist_offsets, user, L_cap, out, stream=None):
    _check("genrank_debug_mask", lib().genrank_debug_mask(
        ctypes.byref(batch), _p(hist_offsets), user, L_cap, _p(out), _stream(stream)))
