"""Pins for the oracle's attention variants (no GPU): the fully visible history mask
([GR-zh] section 1.3.1, the T5-style mask over the historical positions) and the bucketed
time term of the bias ([GR-zh] section 1.4.2, -m_t bucket(t_i - t_j)).

Each pin reduces a variant to something fixed independently: torch's attention without a
mask, a two-key closed form, the raw-seconds bias when the buckets are the integers, no
time term when every edge lies above every gap, and the invariance of candidate rows."""
import math

import numpy as np
import pytest
import torch

import oracle


def _qkv(L, H, dh, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((L, H, dh)) for _ in range(3)]


def _t(a):
    return torch.from_numpy(a).permute(1, 0, 2).contiguous()


def test_full_history_zero_slopes_is_unmasked_softmax():
    N, H, dh = 9, 2, 8
    q, k, v = _qkv(N, H, dh, 1)
    pos, tau = np.arange(N), np.arange(N, dtype=np.float64) * 5
    o, _ = oracle.attn_fwd_user(q, k, v, pos, tau, [0.0] * H, [0.0] * H, N, 0, history="full")
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v))
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def test_full_history_mask_keeps_candidate_rows():
    full, causal = oracle.attention_mask(5, 3, "full"), oracle.attention_mask(5, 3)
    assert full[:5, :5].all() and not full[:5, 5:].any()
    assert np.array_equal(full[5:], causal[5:])


def test_full_history_two_keys_closed_form():
    """The first query sees the later key with the same bias as the reverse pair:
    -s |p_0 - p_1| - s' |tau_0 - tau_1| (distance, not signed difference)."""
    H, dh = 1, 4
    q, k, v = _qkv(2, H, dh, 2)
    pos, tau = np.array([0, 1]), np.array([0.0, 30.0])
    sp, st = 0.5, 0.01
    o, lse = oracle.attn_fwd_user(q, k, v, pos, tau, [sp], [st], 2, 0, history="full")
    s0 = q[0, 0] @ k[0, 0] / 2.0
    s1 = q[0, 0] @ k[1, 0] / 2.0 - sp * 1 - st * 30
    e0, e1 = math.exp(s0), math.exp(s1)
    assert np.allclose(o[0, 0], (e0 * v[0, 0] + e1 * v[1, 0]) / (e0 + e1), atol=1e-12)
    assert abs(lse[0, 0] - math.log(e0 + e1)) < 1e-12


def test_candidate_rows_do_not_depend_on_history_mask():
    N, m, H, dh = 6, 3, 2, 8
    q, k, v = _qkv(N + m, H, dh, 3)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.array([0, 0, 4, 9, 9, 20, 31, 31, 31], dtype=np.float64)
    a, _ = oracle.attn_fwd_user(q, k, v, pos, tau, [0.3, 0.1], [0.02, 0.05], N, m)
    b, _ = oracle.attn_fwd_user(q, k, v, pos, tau, [0.3, 0.1], [0.02, 0.05], N, m, history="full")
    assert np.array_equal(a[N:], b[N:])
    assert not np.allclose(a[:N - 1], b[:N - 1])


def test_time_bucket_counts_edges_at_or_below():
    bounds = [1, 2, 4, 8, 8, 30]
    assert oracle.time_bucket(np.array([0, 1, 3, 7, 8, 29, 30, 1000]), bounds).tolist() == [0, 1, 2, 3, 5, 5, 6, 6]


@pytest.mark.parametrize("history", ["causal", "full"])
def test_integer_buckets_reduce_to_seconds(history):
    """Edges 1, 2, ..., K make bucket(g) = g for g <= K: the bucketed bias equals the
    raw-seconds bias when every gap is at most K."""
    N, m, H, dh = 7, 2, 2, 8
    q, k, v = _qkv(N + m, H, dh, 4)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.array([0, 1, 1, 3, 6, 6, 10, 12, 12], dtype=np.float64)
    raw = oracle.attn_fwd_user(q, k, v, pos, tau, [0.2, 0.05], [0.1, 0.3], N, m, history)
    bkt = oracle.attn_fwd_user(q, k, v, pos, tau, [0.2, 0.05], [0.1, 0.3], N, m, history,
                               time_bounds=np.arange(1, 40))
    assert np.allclose(raw[0], bkt[0], atol=1e-12) and np.allclose(raw[1], bkt[1], atol=1e-12)


def test_edges_above_every_gap_remove_the_time_term():
    N, m, H, dh = 5, 2, 1, 8
    q, k, v = _qkv(N + m, H, dh, 5)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.array([0, 50, 60, 400, 900, 1200, 1200], dtype=np.float64)
    a = oracle.attn_fwd_user(q, k, v, pos, tau, [0.2], [0.0], N, m)
    b = oracle.attn_fwd_user(q, k, v, pos, tau, [0.2], [0.7], N, m, time_bounds=[10 ** 6])
    assert np.allclose(a[0], b[0], atol=1e-12)


def test_bucketed_bias_gradients_by_finite_differences():
    """The backward of the variants against central differences of the forward."""
    N, m, H, dh = 4, 2, 1, 4
    q, k, v = _qkv(N + m, H, dh, 6)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.array([0, 2, 5, 40, 41, 41], dtype=np.float64)
    args = dict(history="full", time_bounds=[1, 3, 10, 30])
    do = np.random.default_rng(7).standard_normal(q.shape)
    dq, dk, dv = oracle.attn_bwd_user(q, k, v, do, pos, tau, [0.3], [0.2], N, m, **args)
    f = lambda qq, kk, vv: float((oracle.attn_fwd_user(qq, kk, vv, pos, tau, [0.3], [0.2], N, m, **args)[0]
                                  * do).sum())
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in [(0, 0, 1), (3, 0, 2), (5, 0, 0)]:
            plus = [x.copy() for x in (q, k, v)]
            minus = [x.copy() for x in (q, k, v)]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num = (f(*plus) - f(*minus)) / (2 * eps)
            assert abs(num - grad[idx]) < 1e-6, (which, idx)
