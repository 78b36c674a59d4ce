"""Pins for the oracle's hand-derived backward pass (no GPU): central finite differences
in float64, plus torch autograd on the CPU as a second, independent check."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from common import oracle_geom, oracle_head, oracle_indices, oracle_layers, oracle_tables, tiny_case


def _fd(f, x, eps=1e-6, samples=None, rng=None):
    """Central differences of scalar f at (a sample of) the entries of x."""
    flat = x.reshape(-1)
    ids = range(flat.size) if samples is None else rng.choice(flat.size, samples, replace=False)
    out = {}
    for i in ids:
        old = flat[i]
        flat[i] = old + eps
        fp = f()
        flat[i] = old - eps
        fm = f()
        flat[i] = old
        out[i] = (fp - fm) / (2 * eps)
    return out


def test_attention_backward_finite_differences():
    N, m, H, dh = 6, 3, 2, 4
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((N + m, H, dh)) for _ in range(3))
    w = rng.standard_normal((N + m, H, dh))
    pos = np.array(list(range(N)) + [N] * m)
    tau = np.array([0, 0, 5, 9, 9, 20, 31, 31, 31], np.float64)
    sp, st = [0.5, 0.25], [0.125, 0.0625]

    def loss():
        o, _ = oracle.attn_fwd_user(q, k, v, pos, tau, sp, st, N, m)
        return float((o * w).sum())

    dq, dk, dv = oracle.attn_bwd_user(q, k, v, w, pos, tau, sp, st, N, m)
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for i, g in _fd(loss, arr).items():
            assert abs(grad.reshape(-1)[i] - g) < 1e-7 * max(1.0, abs(g))


def test_rmsnorm_closed_form_and_backward():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 12)) * 3
    y = oracle.rmsnorm(x, np.ones(12), eps=0.0)
    assert np.allclose(np.sqrt((y * y).mean(1)), 1.0, atol=1e-14)
    g = rng.standard_normal(12)
    w = rng.standard_normal((5, 12))
    dx, dg = oracle.rmsnorm_bwd(x, g, w)
    f = lambda: float((oracle.rmsnorm(x, g) * w).sum())
    for i, gi in _fd(f, x).items():
        assert abs(dx.reshape(-1)[i] - gi) < 1e-7
    for i, gi in _fd(f, g).items():
        assert abs(dg[i] - gi) < 1e-7


def test_silu_and_bce_closed_forms():
    a = np.linspace(-4, 4, 17)
    assert np.allclose(oracle.silu(a), a / (1 + np.exp(-a)))
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    eps = 1e-6
    fd = (oracle.silu(a + eps) - oracle.silu(a - eps)) / (2 * eps)
    assert np.allclose(oracle.silu_bwd(a, np.ones_like(a)), fd, atol=1e-8)
    # BCE at logit 0 is log 2 whatever the label; gradient is (sigmoid(z) - y) / n
    z = np.zeros((3, 4))
    y = (np.arange(12).reshape(3, 4) % 2).astype(float)
    assert math.isclose(oracle.bce_loss(z, y), math.log(2.0), rel_tol=1e-15)
    z = np.random.default_rng(2).standard_normal((3, 4)) * 3
    g = oracle.bce_loss_bwd(z, y)
    for i, gi in _fd(lambda: oracle.bce_loss(z, y), z).items():
        assert abs(g.reshape(-1)[i] - gi) < 1e-9


@pytest.mark.parametrize("block", ["attn_only", "prenorm"])
def test_model_backward_finite_differences(block):
    """Loss = BCE(head(model(embed))) on a tiny 2-layer case; every parameter group,
    the embedding tables included, against central differences."""
    cfg, batch, tables, weights = tiny_case(seed=2, N=7, m=3, block=block, layers=2, d=16)
    idx = oracle_indices(cfg, batch, tables)
    tabs = {k: getattr(tables, k).f32().astype(np.float64).copy()
            for k in ("item", "action", "pos", "ri", "rt")}
    layers = [{k: np.asarray(v, np.float64).copy() for k, v in lw.items()} for lw in oracle_layers(weights)]
    head = {k: np.asarray(v, np.float64).copy() for k, v in oracle_head(weights).items()}
    geom = oracle_geom(cfg, batch, idx)
    labels = synth.make_labels(cfg, B=1)

    def loss():
        x = oracle.embed_sum(tabs, batch.hist_items, batch.cand_items, idx)
        _, logits, _ = oracle.model_fwd(x, layers, block, cfg.H, geom, head)
        return oracle.bce_loss(logits, labels)

    x0 = oracle.embed_sum(tabs, batch.hist_items, batch.cand_items, idx)
    xf, logits, caches = oracle.model_fwd(x0, layers, block, cfg.H, geom, head)
    dl = oracle.bce_loss_bwd(logits, labels)
    dx0, lgrads, hgrads = oracle.model_bwd(dl, xf, layers, block, cfg.H, geom, caches, head)
    tgrads = oracle.embed_bwd(dx0, {k: v.shape for k, v in tabs.items()}, batch.hist_items,
                              batch.cand_items, idx)
    rng = np.random.default_rng(0)
    checks = [(tabs[k], tgrads[k]) for k in ("action", "pos", "ri", "rt")]
    checks.append((tabs["item"], tgrads["item"]))
    for li, lw in enumerate(layers):
        for k in lw:
            if k in lgrads[li]:
                checks.append((lw[k], lgrads[li][k]))
    for k in ("w_head", "b_head", "g_final"):
        checks.append((head[k], hgrads[k]))
    for arr, grad in checks:
        for i, g in _fd(loss, arr, samples=min(6, arr.size), rng=rng).items():
            assert abs(grad.reshape(-1)[i] - g) < 1e-7 * max(1.0, abs(g)) + 1e-10, (i, g)


def test_model_backward_matches_torch_autograd():
    cfg, batch, tables, weights = tiny_case(seed=5, N=9, m=4, block="prenorm", layers=2, d=16)
    idx = oracle_indices(cfg, batch, tables)
    geom = oracle_geom(cfg, batch, idx)
    x0 = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    layers = oracle_layers(weights)
    head = oracle_head(weights)
    labels = synth.make_labels(cfg, B=1)
    xf, logits, caches = oracle.model_fwd(x0, layers, "prenorm", cfg.H, geom, head)
    dx0, lgrads, hgrads = oracle.model_bwd(oracle.bce_loss_bwd(logits, labels), xf, layers,
                                           "prenorm", cfg.H, geom, caches, head)

    # the same forward written with torch ops, differentiated by autograd
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    N, m, H, d = batch.total_hist, cfg.m, cfg.H, cfg.d
    allowed = torch.from_numpy(oracle.attention_mask(N, m))
    pos = torch.tensor(idx["pos"], dtype=torch.float64)
    tau = torch.tensor(idx["tau"], dtype=torch.float64)
    sp, st = geom["slopes_pos"], geom["slopes_time"]
    tx = T(x0)
    tl = [{k: T(v) for k, v in lw.items()} for lw in layers]
    th = {k: T(v) for k, v in head.items()}
    rms = lambda x, g: x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-6) * g
    x = tx
    for lw in tl:
        qkv = rms(x, lw["g1"]) @ lw["wqkv"].T
        q, k, v = (qkv[:, i * d:(i + 1) * d].reshape(-1, H, d // H) for i in range(3))
        outs = []
        for h in range(H):
            bias = -sp[h] * (pos[:, None] - pos[None, :]).abs() - st[h] * (tau[:, None] - tau[None, :]).abs()
            s = q[:, h] @ k[:, h].T / math.sqrt(d // H) + bias
            s = s.masked_fill(~allowed, float("-inf"))
            outs.append(torch.softmax(s, -1) @ v[:, h])
        x = x + torch.cat(outs, 1) @ lw["wo"].T
        x = x + torch.nn.functional.silu(rms(x, lw["g2"]) @ lw["w1"].T) @ lw["w2"].T
    lg = rms(x[N:], th["g_final"]) @ th["w_head"].T + th["b_head"]
    torch.nn.functional.binary_cross_entropy_with_logits(lg, torch.from_numpy(labels).double()).backward()
    assert np.allclose(tx.grad.numpy(), dx0, atol=1e-12)
    for li in range(len(tl)):
        for k, tv in tl[li].items():
            assert np.allclose(tv.grad.numpy(), lgrads[li][k], atol=1e-12), k
    for k in ("w_head", "b_head", "g_final"):
        assert np.allclose(th[k].grad.numpy(), hgrads[k], atol=1e-12), k


def test_history_position_loss_finite_differences():
    """The ablation of [GR-zh] section 1.3.1 that also takes the loss at some history
    positions: BCE over the candidate rows plus two history rows, every parameter group
    against central differences.  Dropping the history rows' head gradient, or scattering
    it to the wrong rows, fails this."""
    cfg, batch, tables, weights = tiny_case(seed=4, N=7, m=3, block="prenorm", layers=2, d=16)
    idx = oracle_indices(cfg, batch, tables)
    tabs = {k: getattr(tables, k).f32().astype(np.float64).copy()
            for k in ("item", "action", "pos", "ri", "rt")}
    layers = [{k: np.asarray(v, np.float64).copy() for k, v in lw.items()} for lw in oracle_layers(weights)]
    head = {k: np.asarray(v, np.float64).copy() for k, v in oracle_head(weights).items()}
    geom = oracle_geom(cfg, batch, idx)
    T_h = batch.total_hist
    rows = np.concatenate([np.arange(T_h, T_h + cfg.m), [1, 5]])
    labels = (np.random.default_rng(3).random((rows.size, 4)) < 0.3).astype(np.float64)

    def loss():
        x = oracle.embed_sum(tabs, batch.hist_items, batch.cand_items, idx)
        _, logits, _ = oracle.model_fwd(x, layers, "prenorm", cfg.H, geom, head, loss_rows=rows)
        return oracle.bce_loss(logits, labels)

    x0 = oracle.embed_sum(tabs, batch.hist_items, batch.cand_items, idx)
    xf, logits, caches = oracle.model_fwd(x0, layers, "prenorm", cfg.H, geom, head, loss_rows=rows)
    assert logits.shape == (rows.size, 4)
    dl = oracle.bce_loss_bwd(logits, labels)
    dx0, lgrads, hgrads = oracle.model_bwd(dl, xf, layers, "prenorm", cfg.H, geom, caches, head,
                                           loss_rows=rows)
    tgrads = oracle.embed_bwd(dx0, {k: v.shape for k, v in tabs.items()}, batch.hist_items,
                              batch.cand_items, idx)
    rng = np.random.default_rng(1)
    checks = [(tabs[k], tgrads[k]) for k in ("item", "action", "pos", "ri", "rt")]
    for li, lw in enumerate(layers):
        checks += [(lw[k], lgrads[li][k]) for k in lw if k in lgrads[li]]
    checks += [(head[k], hgrads[k]) for k in ("w_head", "b_head", "g_final")]
    for arr, grad in checks:
        for i, g in _fd(loss, arr, samples=min(6, arr.size), rng=rng).items():
            assert abs(grad.reshape(-1)[i] - g) < 1e-7 * max(1.0, abs(g)) + 1e-10, (i, g)
    # the default is the candidate rows
    _, lc, _ = oracle.model_fwd(x0, layers, "prenorm", cfg.H, geom, head)
    assert np.array_equal(lc, logits[:cfg.m])
