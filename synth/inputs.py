"""Seeded, synthetic GenRank inputs: jagged user histories, candidates, tables, weights.

The production data of "Towards Large-scale Generative Ranking" (Xiaohongshu Explore Feed
logs) is proprietary; these generators stand in for it with the shapes the pages give:
histories of at most 480 actions (page 1, section 1.3 default setup; page 3), "hundreds"
of candidates per request at the ranking stage (page 1, section 1), requests that group
several items under one timestamp (page 1, section 1.4.2, request-index embedding).

Nothing here implements the method: index derivation, bucketing, embedding sums,
attention and the ALiBi slope schedule live separately in the oracle and in the HIP
library. This module only draws random numbers and lays them out.

Row layout shared by every consumer: rows [0, T_h) are history actions, user after user
(jagged by ``hist_offsets``); row ``T_h + u*m + k`` is candidate k of user u.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------------------
# Configurations
# ----------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    index: int               # seed base = 1000 * index
    B: int                   # users per batch
    hist_min: int            # history length drawn uniformly in [hist_min, hist_max]
    hist_max: int
    m: int                   # candidates per user (one request)
    d: int                   # model dim
    H: int                   # heads (head dim = d // H)
    layers: int
    dtype: str               # activation / table dtype: "f32" or "bf16"
    n_item: int
    n_action: int            # real actions; the mask-action row M is row n_action
    n_pos: int
    n_ri: int
    n_rt: int                # time-gap buckets (n_rt - 1 integer boundaries)
    item_dist: str           # "uniform" or "zipf"
    zipf_a: float = 1.1
    block: str = "prenorm"   # "attn_only": embed -> QKV -> attn -> Wo ; "prenorm": full block
    ffn_mult: int = 4
    n_tasks: int = 4         # click, like, finish, share
    slopes_pos: Optional[tuple] = None   # explicit slopes; None = ALiBi schedule for H heads
    slopes_time: Optional[tuple] = None  # explicit slopes; None = slopes_pos * time_ratio
    time_ratio: float = 0.25
    mean_gap_s: float = 60.0
    t0_base: int = 1_700_000_000
    t0_span: int = 86_400
    train: bool = False

    @property
    def dh(self) -> int:
        return self.d // self.H

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny fp32 sanity case: the oracle finishes in milliseconds.
    "tiny_fp32": Config(
        name="tiny_fp32", index=0, B=1, hist_min=16, hist_max=16, m=4, d=32, H=2, layers=1,
        dtype="f32", n_item=1000, n_action=8, n_pos=16, n_ri=8, n_rt=32, item_dist="uniform",
        block="attn_only", slopes_pos=(2.0 ** -1, 2.0 ** -2), slopes_time=(2.0 ** -3, 2.0 ** -4)),
    # Single-layer inference in bf16 (embed-sum + QKV + masked ALiBi attention + out proj).
    "infer_1layer_bf16": Config(
        name="infer_1layer_bf16", index=1, B=256, hist_min=32, hist_max=480, m=128, d=256, H=4,
        layers=1, dtype="bf16", n_item=1_000_000, n_action=16, n_pos=512, n_ri=64, n_rt=64,
        item_dist="zipf", block="attn_only"),
    # Full 4-layer pre-RMSNorm stack with FFN and the 4-logit action head.
    "stack4_bf16": Config(
        name="stack4_bf16", index=2, B=512, hist_min=480, hist_max=480, m=256, d=512, H=8,
        layers=4, dtype="bf16", n_item=1_000_000, n_action=16, n_pos=512, n_ri=64, n_rt=64,
        item_dist="zipf", block="prenorm"),
    # Training step: 2 layers, BCE on the 4 action logits at candidate positions only.
    "train2_bf16": Config(
        name="train2_bf16", index=3, B=128, hist_min=64, hist_max=480, m=32, d=256, H=4,
        layers=2, dtype="bf16", n_item=1_000_000, n_action=16, n_pos=512, n_ri=64, n_rt=64,
        item_dist="zipf", block="prenorm", train=True),
    # HSTU-style interleaved comparison on the single-layer inference data.
    "hstu_interleaved": Config(
        name="hstu_interleaved", index=4, B=256, hist_min=32, hist_max=480, m=128, d=256, H=4,
        layers=1, dtype="bf16", n_item=1_000_000, n_action=16, n_pos=512, n_ri=64, n_rt=64,
        item_dist="zipf", block="attn_only"),
}
CONFIGS["C0"] = CONFIGS["tiny_fp32"]
CONFIGS["C1"] = CONFIGS["infer_1layer_bf16"]
CONFIGS["C2"] = CONFIGS["stack4_bf16"]
CONFIGS["C3"] = CONFIGS["train2_bf16"]
CONFIGS["C4"] = CONFIGS["hstu_interleaved"]


def make_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# ----------------------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even, as torch and the hardware do)
# ----------------------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


class Stored:
    """A parameter array as the GPU stores it: f32, or bf16 bit patterns."""

    def __init__(self, values_f32: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = f32_to_bf16_bits(values_f32)
            self.shape = self.bits.shape
        elif dtype == "f32":
            self.bits = None
            self._f32 = np.ascontiguousarray(values_f32, dtype=np.float32)
            self.shape = self._f32.shape
        else:
            raise ValueError(dtype)

    @classmethod
    def from_bits(cls, bits: np.ndarray) -> "Stored":
        obj = cls.__new__(cls)
        obj.dtype = "bf16"
        obj.bits = bits
        obj.shape = bits.shape
        return obj

    def f32(self, rows=None) -> np.ndarray:
        """Stored values as float32 (optionally only some rows)."""
        if self.dtype == "f32":
            return self._f32 if rows is None else self._f32[rows]
        b = self.bits if rows is None else self.bits[rows]
        return bf16_bits_to_f32(b)

    def raw(self) -> np.ndarray:
        """The storage array (uint16 bits for bf16, float32 for f32)."""
        return self.bits if self.dtype == "bf16" else self._f32


# ----------------------------------------------------------------------------------------
# Batch: jagged histories + candidates of one request per user
# ----------------------------------------------------------------------------------------


@dataclass
class Batch:
    B: int
    m: int
    hist_offsets: np.ndarray   # int32 [B+1]
    hist_items: np.ndarray     # int32 [T_h]
    hist_actions: np.ndarray   # int32 [T_h]
    hist_ts: np.ndarray        # int64 [T_h], seconds, non-decreasing per user
    cand_items: np.ndarray     # int32 [B*m]
    req_ts: np.ndarray         # int64 [B], request time of the candidates (> last history ts)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.hist_offsets).astype(np.int64)

    @property
    def total_hist(self) -> int:
        return int(self.hist_offsets[-1])

    @property
    def max_hist(self) -> int:
        return int(self.lengths.max()) if self.B > 0 else 0

    @property
    def total_rows(self) -> int:
        return self.total_hist + self.B * self.m

    def subset(self, users) -> "Batch":
        """A new batch made of the given users (in that order)."""
        users = list(users)
        offs = [0]
        items, acts, ts, cands, req = [], [], [], [], []
        for u in users:
            a, b = int(self.hist_offsets[u]), int(self.hist_offsets[u + 1])
            items.append(self.hist_items[a:b])
            acts.append(self.hist_actions[a:b])
            ts.append(self.hist_ts[a:b])
            offs.append(offs[-1] + (b - a))
            cands.append(self.cand_items[u * self.m:(u + 1) * self.m])
            req.append(self.req_ts[u])
        cat = lambda xs, dt: (np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt))
        return Batch(B=len(users), m=self.m, hist_offsets=np.asarray(offs, np.int32),
                     hist_items=cat(items, np.int32), hist_actions=cat(acts, np.int32),
                     hist_ts=cat(ts, np.int64), cand_items=cat(cands, np.int32),
                     req_ts=np.asarray(req, np.int64))


_ZIPF_CDF = {}


def _zipf_cdf(n: int, a: float) -> np.ndarray:
    key = (n, a)
    if key not in _ZIPF_CDF:
        w = np.arange(1, n + 1, dtype=np.float64) ** (-a)
        c = np.cumsum(w)
        _ZIPF_CDF[key] = c / c[-1]
    return _ZIPF_CDF[key]


def _draw_items(rng, cfg: Config, k: int) -> np.ndarray:
    if cfg.item_dist == "uniform":
        return rng.integers(0, cfg.n_item, size=k).astype(np.int32)
    if cfg.item_dist == "zipf":
        # frequency-ordered vocabulary: id = Zipf rank - 1
        u = rng.random(k)
        return np.minimum(np.searchsorted(_zipf_cdf(cfg.n_item, cfg.zipf_a), u, side="right"),
                          cfg.n_item - 1).astype(np.int32)
    raise ValueError(cfg.item_dist)


def _user_events(rng, cfg: Config, n: int):
    """Timestamps of n history actions: requests are runs of 1..4 items sharing one
    integer timestamp; gaps between requests are max(1, round(Exp(mean_gap_s)))."""
    t0 = cfg.t0_base + int(rng.integers(0, cfg.t0_span + 1))
    runs = rng.integers(1, 5, size=max(n, 1))
    gaps = np.maximum(1, np.rint(rng.exponential(cfg.mean_gap_s, size=max(n, 1)))).astype(np.int64)
    req_start = np.cumsum(runs) - runs           # first item index of each request
    req_time = t0 + np.concatenate([[0], np.cumsum(gaps[:-1])])
    req_of_item = np.searchsorted(req_start, np.arange(n), side="right") - 1
    ts = req_time[req_of_item].astype(np.int64)
    last = int(ts[-1]) if n > 0 else t0
    req_ts = last + max(1, int(round(rng.exponential(cfg.mean_gap_s))))
    if n == 0:
        req_ts = t0
    return ts, req_ts


def make_batch(cfg: Config, seed: Optional[int] = None, B: Optional[int] = None,
               lengths: Optional[np.ndarray] = None) -> Batch:
    """Seeded batch.  Each user draws from its own stream (seed, user), so the first k
    users of a batch do not depend on B."""
    seed = 1000 * cfg.index if seed is None else seed
    B = cfg.B if B is None else B
    offs = [0]
    items, acts, ts_all, cands, reqs = [], [], [], [], []
    for u in range(B):
        rng = np.random.default_rng([seed, u])
        n = int(rng.integers(cfg.hist_min, cfg.hist_max + 1))
        if lengths is not None:
            n = int(lengths[u])
        ts, req = _user_events(rng, cfg, n)
        items.append(_draw_items(rng, cfg, n))
        acts.append(rng.integers(0, cfg.n_action, size=n).astype(np.int32))
        cands.append(_draw_items(rng, cfg, cfg.m))
        ts_all.append(ts)
        reqs.append(req)
        offs.append(offs[-1] + n)
    cat = lambda xs, dt: (np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt))
    return Batch(B=B, m=cfg.m, hist_offsets=np.asarray(offs, np.int32),
                 hist_items=cat(items, np.int32), hist_actions=cat(acts, np.int32),
                 hist_ts=cat(ts_all, np.int64), cand_items=cat(cands, np.int32),
                 req_ts=np.asarray(reqs, np.int64))


def make_labels(cfg: Config, B: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """Binary action labels, Bernoulli(0.1), float32 [B*m, n_tasks]."""
    seed = 1000 * cfg.index + 2 if seed is None else seed
    B = cfg.B if B is None else B
    rng = np.random.default_rng(seed)
    return (rng.random((B * cfg.m, cfg.n_tasks)) < 0.1).astype(np.float32)


# ----------------------------------------------------------------------------------------
# Tables and weights
# ----------------------------------------------------------------------------------------


def rt_boundaries(n_rt: int, top_log2: int = 24) -> np.ndarray:
    """Integer lower edges (seconds) of the time-gap buckets 1..n_rt-1, log-spaced from
    1 s to 2**top_log2 s; bucket 0 is reserved for "no earlier request"."""
    nb = n_rt - 1
    b = np.empty(nb, np.int64)
    for k in range(nb):
        v = int(round(2.0 ** (top_log2 * k / max(nb - 1, 1))))
        b[k] = v if k == 0 else max(int(b[k - 1]) + 1, v)
    return b


@dataclass
class Tables:
    item: Stored      # psi   [n_item, d]
    action: Stored    # phi   [n_action + 1, d]; row n_action is the mask-action embedding M
    pos: Stored       # Omega_pe [n_pos, d]
    ri: Stored        # Omega_ri [n_ri, d]
    rt: Stored        # Omega_rt [n_rt, d]
    rt_bounds: np.ndarray  # int64 [n_rt - 1]


def _normal_stored(rng, shape, std, dtype, chunk_rows=65536) -> Stored:
    rows = shape[0]
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"storage dtype must be 'f32' or 'bf16', not {dtype!r}")
    if dtype == "f32":
        return Stored(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), "f32")
    bits = np.empty(shape, np.uint16)
    for a in range(0, rows, chunk_rows):
        b = min(rows, a + chunk_rows)
        blk = rng.standard_normal((b - a,) + tuple(shape[1:]), dtype=np.float32) * np.float32(std)
        bits[a:b] = f32_to_bf16_bits(blk)
    return Stored.from_bits(bits)


def make_tables(cfg: Config, seed: Optional[int] = None, n_item: Optional[int] = None) -> Tables:
    seed = 1000 * cfg.index + 1 if seed is None else seed
    rng = np.random.default_rng(seed)
    d = cfg.d
    n_item = cfg.n_item if n_item is None else n_item
    small = np.random.default_rng([seed, 7])
    return Tables(
        item=_normal_stored(rng, (n_item, d), 0.02, cfg.dtype),
        action=_normal_stored(small, (cfg.n_action + 1, d), 0.02, cfg.dtype),
        pos=_normal_stored(small, (cfg.n_pos, d), 0.02, cfg.dtype),
        ri=_normal_stored(small, (cfg.n_ri, d), 0.02, cfg.dtype),
        rt=_normal_stored(small, (cfg.n_rt, d), 0.02, cfg.dtype),
        rt_bounds=rt_boundaries(cfg.n_rt),
    )


@dataclass
class LayerWeights:
    wqkv: Stored      # [3d, d]: rows 0..d-1 -> Q, d..2d-1 -> K, 2d..3d-1 -> V (y = x W^T)
    wo: Stored        # [d, d]
    w1: Optional[Stored]   # [f*d, d]
    w2: Optional[Stored]   # [d, f*d]
    g1: np.ndarray    # f32 [d] RMSNorm gain before attention
    g2: np.ndarray    # f32 [d] RMSNorm gain before the FFN


@dataclass
class Weights:
    layers: list
    g_final: np.ndarray    # f32 [d]
    w_head: np.ndarray     # f32 [n_tasks, d]
    b_head: np.ndarray     # f32 [n_tasks]


def make_weights(cfg: Config, seed: Optional[int] = None, head_std: Optional[float] = None) -> Weights:
    seed = 1000 * cfg.index + 3 if seed is None else seed
    d, f = cfg.d, cfg.ffn_mult
    layers = []
    for li in range(cfg.layers):
        rng = np.random.default_rng([seed, li])
        wqkv = _normal_stored(rng, (3 * d, d), 0.02, cfg.dtype)
        wo = _normal_stored(rng, (d, d), 0.02, cfg.dtype)
        if cfg.block == "prenorm":
            w1 = _normal_stored(rng, (f * d, d), 0.02, cfg.dtype)
            w2 = _normal_stored(rng, (d, f * d), 0.02, cfg.dtype)
        else:
            w1 = w2 = None
        layers.append(LayerWeights(wqkv=wqkv, wo=wo, w1=w1, w2=w2,
                                   g1=np.ones(d, np.float32), g2=np.ones(d, np.float32)))
    rng = np.random.default_rng([seed, 1000])
    hs = (1.0 / np.sqrt(d)) if head_std is None else head_std
    w_head = (rng.standard_normal((cfg.n_tasks, d)) * hs).astype(np.float32)
    b_head = (rng.standard_normal(cfg.n_tasks) * 0.02).astype(np.float32)
    return Weights(layers=layers, g_final=np.ones(d, np.float32), w_head=w_head, b_head=b_head)


def normal_array(shape, std=1.0, seed=0, dtype="f32") -> Stored:
    """A seeded N(0, std) array in storage form (used for standalone kernel inputs)."""
    return _normal_stored(np.random.default_rng(seed), tuple(shape), std, dtype)
