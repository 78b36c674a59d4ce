"""Pins for the oracle's masked ALiBi attention (no GPU).

Pins used: the pages' slope example and mask example; textbook special cases checked with
torch's scaled_dot_product_attention in float64 on the CPU (a library routine the oracle
does not use); closed forms for two-key cases; and the invariants the pages state
(candidate-alone equivalence, independence between candidates, causal history)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from common import oracle_geom, oracle_indices, oracle_layers, oracle_tables, tiny_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkv(L, H, dh, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((L, H, dh)) * scale for _ in range(3)]


def test_slopes_h8_golden():
    with open(os.path.join(GOLDEN, "alibi_slopes_h8.json")) as f:
        g = json.load(f)
    assert np.array_equal(oracle.alibi_slopes(g["H"]), np.array(g["slopes"]))


def test_mask_worked_example():
    # one history item and two candidates: candidate 1 must not see candidate 2 and
    # vice versa; both see the history item (and themselves)
    assert oracle.attention_mask(1, 2).astype(int).tolist() == [[1, 0, 0], [1, 1, 0], [1, 0, 1]]
    m = oracle.attention_mask(5, 3)
    assert m[:5, :5].astype(int).tolist() == np.tril(np.ones((5, 5), int)).tolist()
    assert not m[:5, 5:].any()
    assert np.array_equal(m[5:, 5:], np.eye(3, dtype=bool))
    assert m[5:, :5].all()


@pytest.mark.parametrize("N,m", [(7, 3), (0, 4), (9, 0), (1, 1)])
def test_zero_slopes_is_textbook_masked_softmax(N, m):
    H, dh = 2, 8
    L = N + m
    q, k, v = _rand_qkv(L, H, dh, seed=N * 10 + m)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.arange(L, dtype=np.float64) * 3
    o, _ = oracle.attn_fwd_user(q, k, v, pos, tau, [0.0] * H, [0.0] * H, N, m)
    mask = torch.from_numpy(oracle.attention_mask(N, m))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
    if m == 0:
        ref2 = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
        assert np.allclose(o, ref2.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def test_no_history_candidate_returns_its_value():
    q, k, v = _rand_qkv(4, 2, 8, seed=3)
    o, lse = oracle.attn_fwd_user(q, k, v, [0] * 4, [0.0] * 4, [0.5, 0.25], [0.1, 0.2], 0, 4)
    assert np.allclose(o, v, atol=1e-15)


def test_two_key_closed_form_bias_terms():
    """q = 0, so the weights come from the biases alone: history row 1 sees keys 0 and 1
    with bias -s*1 - s'*(tau_1 - tau_0) and 0."""
    H, dh = 2, 4
    q = np.zeros((2, H, dh))
    k = np.random.default_rng(1).standard_normal((2, H, dh))
    v = np.random.default_rng(2).standard_normal((2, H, dh))
    sp, st = [0.5, 0.25], [0.125, 0.0625]
    tau = np.array([0.0, 12.0])
    o, lse = oracle.attn_fwd_user(q, k, v, [0, 1], tau, sp, st, 2, 0)
    for h in range(H):
        b0 = -sp[h] * 1 - st[h] * 12.0
        w0 = math.exp(b0) / (math.exp(b0) + 1.0)
        assert np.allclose(o[1, h], w0 * v[0, h] + (1 - w0) * v[1, h], atol=1e-14)
        assert np.isclose(lse[1, h], math.log(math.exp(b0) + 1.0), atol=1e-14)
        assert np.allclose(o[0, h], v[0, h], atol=1e-15)


def test_score_scale_is_one_over_sqrt_head_dim():
    dh = 16
    q = np.zeros((2, 1, dh))
    k = np.zeros((2, 1, dh))
    v = np.zeros((2, 1, dh))
    q[1, 0, 0] = 3.0
    k[0, 0, 0] = 1.0      # q1.k0 = 3, q1.k1 = 0
    v[0, 0, 0] = 1.0
    o, _ = oracle.attn_fwd_user(q, k, v, [0, 0], [0.0, 0.0], [0.0], [0.0], 2, 0)
    w0 = math.exp(3.0 / 4.0) / (math.exp(3.0 / 4.0) + 1.0)
    assert np.isclose(o[1, 0, 0], w0, atol=1e-15)


def test_lse_normalises_the_row():
    N, m, H, dh = 6, 3, 2, 8
    q, k, v = _rand_qkv(N + m, H, dh, seed=5)
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.cumsum(np.arange(N + m)).astype(np.float64)
    sp, st = [0.5, 0.25], [0.01, 0.02]
    _, lse = oracle.attn_fwd_user(q, k, v, pos, tau, sp, st, N, m)
    allowed = oracle.attention_mask(N, m)
    for h in range(H):
        for i in range(N + m):
            s = [q[i, h] @ k[j, h] / math.sqrt(dh) - sp[h] * abs(pos[i] - pos[j]) - st[h] * abs(tau[i] - tau[j])
                 for j in range(N + m) if allowed[i, j]]
            assert np.isclose(sum(math.exp(x - lse[i, h]) for x in s), 1.0, atol=1e-12)


def test_separable_bias_identity():
    """On allowed pairs p_i >= p_j and tau_i >= tau_j, so the bias is u_i + v_j with
    v_j = s p_j + s' tau_j; softmax drops the row constant u_i.  Attention with only the
    column term must equal the literal form (used by the GPU kernel)."""
    N, m, H, dh = 11, 4, 2, 8
    q, k, v = _rand_qkv(N + m, H, dh, seed=9)
    pos = np.array(list(range(N)) + [N] * m, np.float64)
    tau = np.concatenate([np.sort(np.random.default_rng(0).integers(0, 300, N)), [320] * m]).astype(np.float64)
    sp, st = np.array([0.5, 0.25]), np.array([0.125, 0.0625])
    o, _ = oracle.attn_fwd_user(q, k, v, pos, tau, sp, st, N, m)
    allowed = oracle.attention_mask(N, m)
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(dh) + (sp[h] * pos + st[h] * tau)[None, :]
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.allclose(p @ v[:, h], o[:, h], atol=1e-12)


# ---------------------------------------------------------------- invariants on the pages


def _layer_outputs(cfg, batch, tables, weights):
    idx = oracle_indices(cfg, batch, tables)
    x = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    geom = oracle_geom(cfg, batch, idx)
    y, _, _ = oracle.model_fwd(x, oracle_layers(weights), cfg.block, cfg.H, geom)
    return x, y


@pytest.mark.parametrize("block", ["attn_only", "prenorm"])
def test_candidate_alone_equivalence(block):
    """Scoring m candidates together equals appending each candidate alone
    ([GR-note]: predictions equivalent to appending each candidate singly)."""
    cfg, batch, tables, weights = tiny_case(seed=4, block=block)
    x, y = _layer_outputs(cfg, batch, tables, weights)
    T_h = batch.total_hist
    cfg1 = cfg.replace(m=1)
    for k in range(cfg.m):
        b1 = synth.Batch(B=1, m=1, hist_offsets=batch.hist_offsets, hist_items=batch.hist_items,
                         hist_actions=batch.hist_actions, hist_ts=batch.hist_ts,
                         cand_items=batch.cand_items[k:k + 1], req_ts=batch.req_ts)
        x1, y1 = _layer_outputs(cfg1, b1, tables, weights)
        assert np.allclose(x1[T_h], x[T_h + k], atol=1e-15)
        assert np.allclose(y1[T_h], y[T_h + k], atol=1e-13)
        assert np.allclose(y1[:T_h], y[:T_h], atol=1e-13)


def test_candidate_permutation_and_history_independence():
    cfg, batch, tables, weights = tiny_case(seed=6, block="prenorm")
    _, y = _layer_outputs(cfg, batch, tables, weights)
    T_h = batch.total_hist
    perm = np.array([2, 0, 3, 1])
    bp = synth.Batch(B=1, m=cfg.m, hist_offsets=batch.hist_offsets, hist_items=batch.hist_items,
                     hist_actions=batch.hist_actions, hist_ts=batch.hist_ts,
                     cand_items=batch.cand_items[perm], req_ts=batch.req_ts)
    _, yp = _layer_outputs(cfg, bp, tables, weights)
    assert np.allclose(yp[T_h:], y[T_h:][perm], atol=1e-13)
    # history rows do not depend on the candidates at all
    other = synth.Batch(B=1, m=cfg.m, hist_offsets=batch.hist_offsets, hist_items=batch.hist_items,
                        hist_actions=batch.hist_actions, hist_ts=batch.hist_ts,
                        cand_items=(batch.cand_items + 17) % cfg.n_item, req_ts=batch.req_ts + 1000)
    _, yo = _layer_outputs(cfg, other, tables, weights)
    assert np.allclose(yo[:T_h], y[:T_h], atol=0)


def test_history_is_causal():
    """Changing history action s changes no output row before s."""
    cfg, batch, tables, weights = tiny_case(seed=8, block="prenorm")
    _, y = _layer_outputs(cfg, batch, tables, weights)
    s = 9
    acts = batch.hist_actions.copy()
    acts[s] = (acts[s] + 1) % cfg.n_action
    b2 = synth.Batch(B=1, m=cfg.m, hist_offsets=batch.hist_offsets, hist_items=batch.hist_items,
                     hist_actions=acts, hist_ts=batch.hist_ts, cand_items=batch.cand_items,
                     req_ts=batch.req_ts)
    _, y2 = _layer_outputs(cfg, b2, tables, weights)
    assert np.array_equal(y2[:s], y[:s])
    assert not np.allclose(y2[s], y[s])
    # the time bias makes the effect on candidates small, but it must be there
    assert np.abs(y2[batch.total_hist:] - y[batch.total_hist:]).max() > 0


def test_multi_user_batch_equals_users_alone():
    cfg = synth.make_config("tiny_fp32", B=3, hist_min=0, hist_max=9)
    batch = synth.make_batch(cfg, seed=21, lengths=np.array([5, 0, 9]))
    tables, weights = synth.make_tables(cfg), synth.make_weights(cfg)
    _, y = _layer_outputs(cfg, batch, tables, weights)
    for u in range(3):
        bu = batch.subset([u])
        _, yu = _layer_outputs(cfg.replace(B=1), bu, tables, weights)
        rows = oracle.user_rows(batch.hist_offsets, cfg.m, u)
        assert np.allclose(yu, y[rows], atol=1e-14)
