"""Algorithmic work of the GenRank hot path, for measurement (no GPU needed).

Attention: user u with N history actions and m candidates has N(N+1)/2 causal history
pairs plus m(N+1) candidate pairs (all history + itself); each pair costs 2*d flops for
QK^T and 2*d for PV over all heads (4*d per pair).  Candidate x candidate pairs other than
the diagonal are not work: the mask removes them.
"""
from __future__ import annotations

import numpy as np


def attention_pairs(lengths, m: int, full_history: bool = False) -> int:
    """Allowed (query, key) pairs: a causal (or, with ``full_history``, fully visible)
    history, and m candidates that each see the history and themselves."""
    n = np.asarray(lengths, dtype=np.int64)
    hist = (n * n).sum() if full_history else (n * (n + 1) // 2).sum()
    return int(hist + m * (n + 1).sum())


def attention_fwd_flops(lengths, m: int, d: int, full_history: bool = False) -> int:
    return 4 * d * attention_pairs(lengths, m, full_history)


def attention_hbm_floor_bytes(rows: int, d: int, elem: int = 2, lse: bool = True, H: int = 1) -> int:
    """Read Q, K, V once and write O once (+ the f32 log-sum-exp)."""
    return rows * d * elem * 4 + (rows * H * 4 if lse else 0)


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def gather_compulsory_bytes(rows: int, d: int, elem: int, unique_items: int, small_rows: int,
                            index_bytes: int) -> int:
    """Embedding gather-sum: one write of every output row, each distinct item row read once,
    the small tables read once, and the per-row index inputs."""
    return rows * d * elem + unique_items * d * elem + small_rows * d * elem + index_bytes


def gather_logical_bytes(rows: int, d: int, elem: int, index_bytes: int) -> int:
    """Five table rows read and one row written per token."""
    return rows * d * elem * 6 + index_bytes


def interleaved_tokens(n_c: int, m: int = 0) -> int:
    """HSTU-style interleaving: one token per item and one per action, then candidates."""
    return 2 * n_c + m


def action_oriented_tokens(n_c: int, m: int = 0) -> int:
    return n_c + m


def attention_bwd_flops(lengths, m: int, d: int, recompute: bool = False, full_history: bool = False) -> int:
    """Backward over the allowed pairs: dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q
    (2 d flops each per pair, twice the forward); with ``recompute`` also S = Q K^T again
    (2.5 times the forward)."""
    per_pair = 8 * d + (2 * d if recompute else 0)
    return per_pair * attention_pairs(lengths, m, full_history)


def attention_bwd_hbm_floor_bytes(rows: int, d: int, H: int, elem: int = 2) -> int:
    """Read Q, K, V, O, dO and the log-sum-exp once, write dQ, dK, dV once, and write and
    read the per-row D = rowsum(dO * O) once."""
    return rows * d * elem * 8 + rows * H * 4 * 3
