"""Helpers that turn synthetic inputs into the oracle's plain arrays (no arithmetic of
the method lives here)."""
import numpy as np

import oracle
import synth


class RowView:
    """Row access to a stored table, converting only the rows asked for to float32."""

    def __init__(self, stored):
        self.stored = stored
        self.shape = stored.shape

    def __getitem__(self, ids):
        return self.stored.f32(np.asarray(ids))


def oracle_tables(tables):
    return {k: RowView(getattr(tables, k)) for k in ("item", "action", "pos", "ri", "rt")}


def oracle_slopes(cfg):
    sp = np.asarray(cfg.slopes_pos, np.float64) if cfg.slopes_pos is not None else oracle.alibi_slopes(cfg.H)
    st = np.asarray(cfg.slopes_time, np.float64) if cfg.slopes_time is not None else sp * cfg.time_ratio
    return sp, st


def oracle_indices(cfg, batch, tables, users=None):
    return oracle.token_indices(batch.hist_offsets, batch.hist_actions, batch.hist_ts,
                                batch.req_ts, batch.m, cfg.n_action, cfg.n_pos, cfg.n_ri,
                                tables.rt_bounds, users=users)


def oracle_layers(weights):
    out = []
    for lw in weights.layers:
        d = {"wqkv": lw.wqkv.f32(), "wo": lw.wo.f32(), "g1": lw.g1, "g2": lw.g2}
        if lw.w1 is not None:
            d["w1"] = lw.w1.f32()
            d["w2"] = lw.w2.f32()
        out.append(d)
    return out


def oracle_head(weights):
    return {"g_final": weights.g_final, "w_head": weights.w_head, "b_head": weights.b_head}


def oracle_geom(cfg, batch, idx):
    sp, st = oracle_slopes(cfg)
    return {"hist_offsets": batch.hist_offsets, "m": batch.m, "pos": idx["pos"],
            "tau": idx["tau"], "slopes_pos": sp, "slopes_time": st}


def tiny_case(seed=0, N=16, m=4, **kw):
    cfg = synth.make_config("tiny_fp32", **kw)
    batch = synth.make_batch(cfg, seed=seed, lengths=np.full(cfg.B, N)) if N is not None else synth.make_batch(cfg, seed=seed)
    if m != cfg.m:
        cfg = cfg.replace(m=m)
        batch = synth.make_batch(cfg, seed=seed, lengths=np.full(cfg.B, N))
    tables = synth.make_tables(cfg)
    weights = synth.make_weights(cfg)
    return cfg, batch, tables, weights
