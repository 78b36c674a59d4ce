"""The oracle's HSTU-interleaved comparison path (learned relative bias read from memory),
pinned to the pages and to the already-pinned ALiBi attention.  No GPU."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_interleaved_layout_matches_the_pages():
    with open(os.path.join(GOLDEN, "sequence_length_cost.json")) as f:
        g = json.load(f)
    n = g["n_c"]
    kind, src, pos = oracle.hstu_sequence(n, 0)
    assert len(kind) == g["interleaved_tokens"]  # item and action tokens, 2 per action
    kind, src, pos = oracle.hstu_sequence(5, 3)
    assert list(kind) == [0, 1] * 5 + [2, 2, 2]
    assert list(src[:10]) == [0, 0, 1, 1, 2, 2, 3, 3, 4, 4] and list(src[10:]) == [0, 1, 2]
    assert list(pos[:10]) == list(range(10)) and list(pos[10:]) == [10, 10, 10]  # shared slot


def test_rab_symmetry_diagonal_and_terms():
    rng = np.random.default_rng(3)
    N, m = 7, 4
    ts = np.cumsum(rng.integers(0, 90, N)) + 1_700_000_000
    t = oracle.hstu_times(ts, ts[-1] + 30, N, m)
    _, _, pos = oracle.hstu_sequence(N, m)
    bounds = synth.rt_boundaries(16)
    pt, tt = rng.standard_normal(4), rng.standard_normal(16)
    rab = oracle.hstu_rab(pos, t, pt, tt, bounds)
    assert np.array_equal(rab, rab.T)
    assert np.allclose(np.diag(rab), pt[0] + tt[0])
    # the position term alone: |p_i - p_j| clamped to the last of 4 rows
    pos_only = oracle.hstu_rab(pos, t, np.arange(4.0), np.zeros(16), bounds)
    assert np.array_equal(pos_only, np.minimum(np.abs(pos[:, None] - pos[None, :]), 3))


def test_rab_time_bucket_agrees_with_token_indices():
    # The time-gap bucket of the embedding indices is pinned (golden vectors); a gap of g
    # seconds between two single-item requests must land in the same bucket here.
    bounds = synth.rt_boundaries(64)
    for g in (1, 2, 3, 59, 60, 61, 600, 3601, 86400, 10 ** 6, 2 ** 24):
        ts = np.array([1_000_000, 1_000_000 + g], np.int64)
        idx = oracle.token_indices(np.array([0, 2], np.int32), np.zeros(2, np.int32), ts,
                                   np.array([ts[-1] + 1], np.int64), 0, 8, 16, 8, bounds)
        t = oracle.hstu_times(ts, ts[-1] + 1, 2, 0)
        _, _, pos = oracle.hstu_sequence(2, 0)
        rab = oracle.hstu_rab(pos, t, np.zeros(4), np.arange(64.0), bounds)
        assert rab[2, 0] == idx["rt"][1], g  # item token of action 1 vs action 0


def test_rab_attention_reduces_to_alibi_attention():
    # With the bias matrix set to the ALiBi bias of the same slots, the HSTU attention is the
    # pinned ALiBi attention over a history of 2N slots.
    rng = np.random.default_rng(11)
    N, m, dh = 9, 5, 16
    L = 2 * N + m
    ts = np.cumsum(rng.integers(0, 50, N)) + 1_700_000_000
    t = oracle.hstu_times(ts, ts[-1] + 20, N, m)
    _, _, pos = oracle.hstu_sequence(N, m)
    tau = (t - t[0]).astype(np.float64)
    sp, st = 0.25, 0.01
    q, k, v = (rng.standard_normal((L, 1, dh)) for _ in range(3))
    rab = -sp * np.abs(pos[:, None] - pos[None, :]) - st * np.abs(tau[:, None] - tau[None, :])
    o1, l1 = oracle.hstu_attn_fwd_user(q, k, v, rab, N, m)
    o2, l2 = oracle.attn_fwd_user(q, k, v, pos, tau, [sp], [st], 2 * N, m)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
