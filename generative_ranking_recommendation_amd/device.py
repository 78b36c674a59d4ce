"""Uploads host arrays to device memory and builds the C structs that point at them.

Inputs are duck-typed: a batch needs ``hist_offsets, hist_items, hist_actions, hist_ts,
cand_items, req_ts, B, m``; a stored parameter needs ``dtype`` ("f32"/"bf16") and ``raw()``
(float32 values, or bf16 bit patterns as uint16).  No arithmetic happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

DTYPE_CODE = {"f32": B.F32, "bf16": B.BF16}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(arr, device, dtype=None):
    a = np.ascontiguousarray(arr if dtype is None else np.asarray(arr, dtype=dtype))
    return torch.from_numpy(a).to(device)


def stored_to_device(stored, device):
    raw = np.ascontiguousarray(stored.raw())
    if stored.dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(raw.astype(np.float32, copy=False)).to(device)


class DeviceInputs:
    """One batch of jagged histories + candidates in device memory."""

    def __init__(self, batch, device="cuda"):
        self.B = int(batch.B)
        self.m = int(batch.m)
        offs = np.asarray(batch.hist_offsets, np.int32)
        self.total_hist = int(offs[-1])
        self.max_hist = int(np.diff(offs).max()) if self.B > 0 else 0
        self.lengths = np.diff(offs).astype(np.int64)
        self.host = batch
        self.hist_offsets = to_device(offs, device)
        self.hist_items = to_device(batch.hist_items, device, np.int32)
        self.hist_actions = to_device(batch.hist_actions, device, np.int32)
        self.hist_ts = to_device(batch.hist_ts, device, np.int64)
        self.cand_items = to_device(batch.cand_items, device, np.int32)
        self.req_ts = to_device(batch.req_ts, device, np.int64)
        self.struct = B.make_inputs(self.hist_offsets, self.hist_items, self.hist_actions,
                                    self.hist_ts, self.cand_items, self.req_ts)

    @property
    def rows(self) -> int:
        return self.total_hist + self.B * self.m


class DeviceTables:
    def __init__(self, tables, device="cuda"):
        self.dtype = tables.item.dtype
        self.item = stored_to_device(tables.item, device)
        self.action = stored_to_device(tables.action, device)
        self.pos = stored_to_device(tables.pos, device)
        self.ri = stored_to_device(tables.ri, device)
        self.rt = stored_to_device(tables.rt, device)
        bounds = np.asarray(tables.rt_bounds, np.int64)
        self.rt_bounds = to_device(bounds if len(bounds) else np.zeros(1, np.int64), device)
        self.d = int(self.item.shape[1])
        self.struct = B.make_tables(self.item, self.action, self.pos, self.ri, self.rt,
                                    self.rt_bounds, int(self.item.shape[0]),
                                    int(self.action.shape[0]) - 1, int(self.pos.shape[0]),
                                    int(self.ri.shape[0]), int(self.rt.shape[0]))


class DeviceLayer:
    """One block's weights on the device plus its ALiBi slopes (host)."""

    def __init__(self, lw, slopes_pos, slopes_time, block, device="cuda", attn_flags=0, time_bounds=None):
        """attn_flags: ATTN_FULL_HISTORY and/or ATTN_TIME_BUCKET; time_bounds: the ascending
        integer bucket edges (seconds) of the bucketed time term."""
        self.block = block
        self.wqkv = stored_to_device(lw.wqkv, device)
        self.wo = stored_to_device(lw.wo, device)
        self.time_bounds = None
        if time_bounds is not None:
            self.time_bounds = torch.as_tensor(np.ascontiguousarray(time_bounds, np.int64)).to(device)
        self.slopes = B.HostSlopes(slopes_pos, slopes_time, attn_flags, self.time_bounds)
        if block == B.BLOCK_PRENORM:
            self.w1 = stored_to_device(lw.w1, device)
            self.w2 = stored_to_device(lw.w2, device)
            self.g1 = to_device(lw.g1, device, np.float32)
            self.g2 = to_device(lw.g2, device, np.float32)
            self.ffn_dim = int(self.w1.shape[0])
        else:
            self.w1 = self.w2 = self.g1 = self.g2 = None
            self.ffn_dim = 0
        self.struct = B.make_layer_weights(self.wqkv, self.wo, self.slopes, block, self.w1, self.w2,
                                           self.g1, self.g2, self.ffn_dim)


class DeviceHead:
    def __init__(self, weights, device="cuda"):
        self.g_final = to_device(weights.g_final, device, np.float32)
        self.w_head = to_device(weights.w_head, device, np.float32)
        self.b_head = to_device(weights.b_head, device, np.float32)
        self.n_tasks = int(self.w_head.shape[0])
