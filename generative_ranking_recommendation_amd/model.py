"""GenRank forward / training step as a chain of C-ABI calls on one HIP stream.

    embed-sum (five tables, fused index derivation)
      -> L blocks (QKV GEMM -> masked ALiBi attention -> output GEMM [-> FFN])
      -> action head at candidate rows -> [BCE at candidates -> backward]

The class owns device weights and cached workspaces; every step runs in libgenrank's
kernels.  Workspaces are allocated once per batch shape, outside any timed region.
"""
from __future__ import annotations

import torch

from . import binding as B
from .device import DTYPE_CODE, TORCH_DTYPE, DeviceHead, DeviceLayer, DeviceTables


class GenRank:
    def __init__(self, tables: DeviceTables, layers: list, H: int, head: DeviceHead = None,
                 device="cuda", resid=None):
        """resid: B.RESID_ACT or B.RESID_F32, the residual stream's element type; by default
        f32 for a bf16 stack of pre-norm blocks (its residual sums are kept in f32, the
        projections' operands in bf16), the activation dtype otherwise."""
        self.tables = tables
        self.layers = layers
        self.head = head
        self.H = H
        self.d = tables.d
        self.dtype = tables.dtype
        self.code = DTYPE_CODE[self.dtype]
        prenorm = bool(layers) and all(lay.block == B.BLOCK_PRENORM for lay in layers)
        if resid is None:
            resid = B.RESID_F32 if (self.dtype == "bf16" and prenorm) else B.RESID_ACT
        self.resid = resid
        self.resid_code = B.F32 if resid == B.RESID_F32 else self.code
        self.device = device
        self._ws = {}

    @classmethod
    def from_host(cls, cfg, tables, weights, slopes_pos, slopes_time, device="cuda", attn_flags=0,
                  time_bounds=None, resid=None):
        block = B.BLOCK_PRENORM if cfg.block == "prenorm" else B.BLOCK_ATTN_ONLY
        dt = DeviceTables(tables, device)
        layers = [DeviceLayer(lw, slopes_pos, slopes_time, block, device, attn_flags, time_bounds)
                  for lw in weights.layers]
        head = DeviceHead(weights, device) if cfg.block == "prenorm" else None
        return cls(dt, layers, cfg.H, head, device, resid)

    # ---------------------------------------------------------------- helpers
    def batch(self, inp) -> B.Batch:
        return B.make_batch(inp.B, inp.m, self.d, self.H, inp.max_hist, inp.total_hist, self.code, self.resid)

    def _buf(self, key, nbytes):
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = t
        return t

    def act(self, rows, cols=None):
        """rows in the activation dtype (projection operands, gradients)"""
        return torch.empty((rows, cols or self.d), dtype=TORCH_DTYPE[self.dtype], device=self.device)

    def resid_rows(self, rows):
        """residual-stream rows (embedding output, block inputs and outputs)"""
        dt = torch.float32 if self.resid == B.RESID_F32 else TORCH_DTYPE[self.dtype]
        return torch.empty((rows, self.d), dtype=dt, device=self.device)

    # ---------------------------------------------------------------- forward
    def embed(self, inp, x_out, stream=None):
        B.genrank_embed_sum(self.batch(inp), inp.struct, self.tables.struct, x_out, stream)

    def layer(self, i, inp, x_in, y_out, save=False, stream=None):
        lay = self.layers[i]
        bt = self.batch(inp)
        nbytes = B.genrank_workspace_size(B.OP_LAYER_FWD, bt, lay.struct)
        ws = self._buf(("fwd", i), nbytes)
        B.genrank_layer_fwd(bt, lay.struct, inp.hist_offsets, inp.hist_ts, inp.req_ts, x_in, y_out,
                            B.FWD_SAVE if save else 0, ws, nbytes, stream)
        return ws

    def forward(self, inp, save=False, stream=None, bufs=None):
        """Returns (x_final, logits or None).  ``bufs`` may pass preallocated
        {"x": [T, d], "y": [T, d], "logits": [B*m, n_tasks]} tensors."""
        T = inp.rows
        bufs = bufs or {}
        x = bufs.get("x") if bufs.get("x") is not None else self.resid_rows(T)
        self.embed(inp, x, stream)
        xs = [x]
        for i in range(len(self.layers)):
            if self.layers[i].block == B.BLOCK_ATTN_ONLY:
                y = bufs.get("y") if bufs.get("y") is not None else self.resid_rows(T)
            else:
                y = x if not save else self.resid_rows(T)
            self.layer(i, inp, x, y, save, stream)
            x = y
            xs.append(x)
        self._xs = xs
        logits = None
        if self.head is not None:
            logits = bufs.get("logits")
            if logits is None:
                logits = torch.empty((inp.B * inp.m, self.head.n_tasks), dtype=torch.float32,
                                     device=self.device)
            B.genrank_head_fwd(self.batch(inp), x, self.head.g_final, self.head.w_head,
                               self.head.b_head, self.head.n_tasks, logits, stream)
        return x, logits

    # ---------------------------------------------------------------- serving with cached history
    def prefill(self, inp, stream=None):
        """Per-block history keys and values of the batch's users, each [T_h, 2d] (keys in
        columns [0, d), values in [d, 2d)).  History rows never depend on candidates, so this
        is a forward over the history rows alone; the top block stops at its key/value
        projection (its history outputs are never read)."""
        T_h = inp.total_hist
        d = self.d
        bh = B.make_batch(inp.B, 0, d, self.H, inp.max_hist, T_h, self.code, self.resid)
        x = self.resid_rows(T_h)
        B.genrank_embed_sum(bh, inp.struct, self.tables.struct, x, stream)
        caches = []
        for i, lay in enumerate(self.layers):
            kv = self.act(T_h, 2 * d)
            nb = B.genrank_workspace_size(B.OP_LAYER_KV, bh, lay.struct)
            B.genrank_layer_kv(bh, lay.struct, x, kv, 2 * d, self._buf(("kv", i), nb), nb, stream)
            caches.append(kv)
            if i + 1 < len(self.layers):
                y = self.resid_rows(T_h)
                nf = B.genrank_workspace_size(B.OP_LAYER_FWD, bh, lay.struct)
                B.genrank_layer_fwd(bh, lay.struct, inp.hist_offsets, inp.hist_ts, inp.req_ts, x, y, 0,
                                    self._buf(("prefill", i), nf), nf, stream)
                x = y
        return caches

    def score(self, inp, caches, stream=None):
        """The candidate rows of ``forward`` from cached history keys and values: returns
        (x [B*m, d] after the last block, logits [B*m, n_tasks] or None)."""
        bt = self.batch(inp)
        Tc = inp.B * inp.m
        d = self.d
        x = self.resid_rows(Tc)
        B.genrank_embed_sum_cand(bt, inp.struct, self.tables.struct, x, stream)
        for i, lay in enumerate(self.layers):
            y = self.resid_rows(Tc) if lay.block == B.BLOCK_ATTN_ONLY else x
            nb = B.genrank_workspace_size(B.OP_LAYER_FWD_CACHED, bt, lay.struct)
            B.genrank_layer_fwd_cached(bt, lay.struct, inp.hist_offsets, inp.hist_ts, inp.req_ts, caches[i],
                                       2 * d, x, y, self._buf(("cached", i), nb), nb, stream)
            x = y
        logits = None
        if self.head is not None:
            bc = B.make_batch(inp.B, inp.m, d, self.H, 0, 0, self.code, self.resid)  # candidate rows only
            logits = torch.empty((Tc, self.head.n_tasks), dtype=torch.float32, device=self.device)
            B.genrank_head_fwd(bc, x, self.head.g_final, self.head.w_head, self.head.b_head, self.head.n_tasks,
                               logits, stream)
        return x, logits

    # ---------------------------------------------------------------- training
    def train_step(self, inp, labels, stream=None, hist_rows=None, hist_labels=None):
        """Forward with saved activations, BCE at candidates, full backward.  Returns
        (loss tensor [1], logits, grads dict of f32 tensors).

        ``hist_rows`` (device int32, distinct history row indices in [0, T_h)) and
        ``hist_labels`` ([len(hist_rows), n_tasks] f32): also take the loss at those history
        positions (the history-position loss ablation); the logits then cover the candidate
        rows followed by the listed history rows, and the BCE is the mean over all of them."""
        x_final, logits = self.forward(inp, save=True, stream=stream)
        bt = self.batch(inp)
        dev, d = self.device, self.d
        n = inp.B * inp.m
        nt = self.head.n_tasks
        nwh = B.genrank_workspace_size(B.OP_HEAD_BWD, bt)
        rows = None
        if hist_rows is not None and hist_rows.numel() > 0:
            rows = torch.cat([torch.arange(inp.total_hist, inp.rows, dtype=torch.int32, device=dev),
                              hist_rows.to(torch.int32)])
            n = int(rows.numel())
            labels = torch.cat([labels, hist_labels])
            logits = torch.empty((n, nt), dtype=torch.float32, device=dev)
            B.genrank_head_fwd_rows(self.resid_code, d, x_final, n, rows, self.head.g_final, self.head.w_head,
                                    self.head.b_head, nt, logits, stream)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        dlogits = torch.empty((n, nt), dtype=torch.float32, device=dev)
        B.genrank_bce_loss(n, nt, logits, labels, loss, dlogits, stream)
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        grads = {"g_final": f32(d), "w_head": f32(nt, d), "b_head": f32(nt)}
        dx = self.act(inp.rows)
        if rows is None:
            B.genrank_head_bwd(bt, x_final, self.head.g_final, self.head.w_head, nt, dlogits, dx,
                               grads["g_final"], grads["w_head"], grads["b_head"],
                               self._buf(("head_bwd",), nwh), nwh, stream)
        else:
            B.genrank_head_bwd_rows(self.resid_code, self.code, d, inp.rows, x_final, n, rows, self.head.g_final,
                                    self.head.w_head, nt, dlogits, dx, grads["g_final"], grads["w_head"],
                                    grads["b_head"], self._buf(("head_bwd",), nwh), nwh, stream)
        grads["layers"] = [None] * len(self.layers)
        for i in range(len(self.layers) - 1, -1, -1):
            lay = self.layers[i]
            lg = {"wqkv": f32(3 * d, d), "wo": f32(d, d)}
            if lay.block == B.BLOCK_PRENORM:
                lg.update(w1=f32(lay.ffn_dim, d), w2=f32(d, lay.ffn_dim), g1=f32(d), g2=f32(d))
            gstruct = B.make_layer_grads(lg["wqkv"], lg["wo"], lg.get("w1"), lg.get("w2"),
                                         lg.get("g1"), lg.get("g2"))
            nb = B.genrank_workspace_size(B.OP_LAYER_BWD, bt, lay.struct)
            wsb = self._buf(("bwd",), nb)
            nf = B.genrank_workspace_size(B.OP_LAYER_FWD, bt, lay.struct)
            B.genrank_layer_bwd(bt, lay.struct, inp.hist_offsets, inp.hist_ts, inp.req_ts,
                                self._xs[i], self._ws[("fwd", i)], dx, dx, gstruct,
                                1 if (i == len(self.layers) - 1 and rows is None) else 0, wsb, nb, stream)
            del nf
            grads["layers"][i] = lg
        # table gradients: the item table's sparse (distinct ids ascending, their rows, the
        # count on the device), the small tables' dense
        t = self.tables
        T = inp.rows
        tg = {k: torch.empty(getattr(t, k).shape, dtype=torch.float32, device=dev)
              for k in ("action", "pos", "ri", "rt")}
        tg["item_ids"] = torch.empty(T, dtype=torch.int32, device=dev)
        tg["item_rows"] = torch.empty((T, d), dtype=torch.float32, device=dev)
        tg["n_items"] = torch.empty(1, dtype=torch.int32, device=dev)
        nwe = B.genrank_workspace_size(B.OP_EMBED_BWD, bt)
        wse = self._buf(("embed_bwd",), nwe)
        B.genrank_embed_bwd(bt, inp.struct, t.struct, dx, tg["item_ids"], tg["item_rows"], tg["n_items"],
                            tg["action"], tg["pos"], tg["ri"], tg["rt"], wse, nwe, stream)
        grads["tables"] = tg
        return loss, logits, grads
