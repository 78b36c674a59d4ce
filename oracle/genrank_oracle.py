"""CPU oracle for GenRank's ranking forward and backward pass.

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, float64 numpy implementation written
from the pages on "Towards Large-scale Generative Ranking" (GenRank, Xiaohongshu).  It is
used by the tests, by ``__graft_entry__.smoke()`` and by the benchmark's CPU-baseline
leg, and by nothing else.  It shares no code with the HIP library and imports nothing from
it.  Every function follows one definition from the pages, cited by page title and
section; where the pages leave a step open the plainest reading is taken and named
("reading:").  There is no blocking, fusion or reordering beyond the definitions.

Page titles used in citations:
  [GR-zh]   "一、 GenRank [2025]" (huaxiaozhuan.com, Chinese paraphrase of the paper)
  [GR-sum]  "Towards Large-scale Generative Ranking" source-linked summary (paperlayer.ai)
  [GR-note] "生成式排序 —— 小红书 GenRank 精读笔记" (wln20.github.io)
  [FR-en]   "The Overall Generative Ranking Paradigm" (fun-rec mdbook, English, ch. 7.2)

Conventions (shared data layout, not shared code):
  * rows [0, T_h) are history actions, user after user, jagged by ``hist_offsets``;
    row ``T_h + u*m + k`` is candidate k of user u;
  * a linear layer with weight ``w`` of shape [out, in] computes ``x @ w.T``;
  * Q/K/V/O are [T, H, dh].

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` except the transformer-block internals (RMSNorm placement, FFN
shape), which the pages do not describe; those are textbook definitions checked only
through the invariants and closed forms listed in the tests.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "alibi_slopes",
    "user_rows",
    "token_indices",
    "embed_sum",
    "attention_mask",
    "time_bucket",
    "attn_fwd_user",
    "attn_fwd",
    "attn_bwd_user",
    "attn_bwd",
    "rmsnorm",
    "rmsnorm_bwd",
    "silu",
    "silu_bwd",
    "layer_fwd",
    "layer_bwd",
    "head_fwd",
    "head_bwd",
    "bce_loss",
    "bce_loss_bwd",
    "model_fwd",
    "model_bwd",
    "embed_bwd",
    "hstu_sequence",
    "hstu_rab",
    "hstu_attn_fwd_user",
    "hstu_times",
    "round_bf16",
]

RMS_EPS = 1e-6


# ----------------------------------------------------------------------------------------
# ALiBi slopes
# ----------------------------------------------------------------------------------------


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes m_h = 2^(-8(h+1)/H), h = 0..H-1.

    [GR-zh] section 1.4.2, the slope formula (second form) and its H = 8 example
    (1/2, 1/4, ..., 1/256)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float64)


# ----------------------------------------------------------------------------------------
# Token indices (position, request index, pre-request time gap)
# ----------------------------------------------------------------------------------------


def user_rows(hist_offsets: np.ndarray, m: int, u: int) -> np.ndarray:
    """Global row numbers of user u's sequence: history in order, then its m candidates."""
    T_h = int(hist_offsets[-1])
    a, b = int(hist_offsets[u]), int(hist_offsets[u + 1])
    return np.concatenate([np.arange(a, b), T_h + u * m + np.arange(m)]).astype(np.int64)


def token_indices(hist_offsets, hist_actions, hist_ts, req_ts, m, n_action, n_pos, n_ri,
                  rt_bounds, users=None):
    """Per-row indices into the five embedding tables, plus ALiBi coordinates.

    For user u with N history actions and m candidates, sequence slot s = 0..N+m-1:
      * action slot: a_s for history; n_action (the mask-action row M) for candidates
        ([GR-zh] section 1.4.1, candidate token e_j = psi(x_j) + m).
      * position p_s = s for history; N for every candidate, since the candidates of one
        request share one position ([GR-zh] section 1.4.2, position embeddings, and its
        example of 100 history items whose 3 candidates all sit at position 101, 1-based;
        reading: 0-based here).  Table slot min(p, n_pos - 1) (reading: clamp).
      * request index = |{t_1..t_s}|, the number of distinct timestamps in the prefix
        ([GR-zh] section 1.4.2, request index embeddings).  For a candidate the prefix is
        the whole history plus the candidate itself (reading: a candidate is scored as if it
        were appended alone, [GR-note]).  Table slot min(ri - 1, n_ri - 1).
      * pre-request gap = t_s - max{t_j in prefix : t_j < t_s}
        ([GR-zh] section 1.4.2, pre-request time embeddings); bucket = #{k : b_k <= gap}
        over the caller's integer boundaries b (reading: the pages do not give bucket();
        bucket 0 means "no earlier request").
      * tau_s = t_s - (user's first timestamp), seconds, used by the time ALiBi term; a
        candidate's time is the request time ``req_ts[u]``.

    Returns a dict of arrays over all T rows (rows of users not in ``users`` stay -1/NaN).
    """
    hist_offsets = np.asarray(hist_offsets, np.int64)
    B = len(hist_offsets) - 1
    T_h = int(hist_offsets[-1])
    T = T_h + B * m
    bounds = [int(b) for b in rt_bounds]
    out = {
        "act": np.full(T, -1, np.int64),
        "pos": np.full(T, -1, np.int64),
        "pe": np.full(T, -1, np.int64),
        "ri": np.full(T, -1, np.int64),
        "ri_slot": np.full(T, -1, np.int64),
        "gap": np.full(T, -1, np.int64),
        "rt": np.full(T, -1, np.int64),
        "tau": np.full(T, np.nan, np.float64),
    }
    for u in (range(B) if users is None else users):
        a, b = int(hist_offsets[u]), int(hist_offsets[u + 1])
        N = b - a
        hist_t = [int(t) for t in hist_ts[a:b]]
        req = int(req_ts[u])
        times = hist_t + [req] * m
        first = times[0]
        rows = user_rows(hist_offsets, m, u)
        for s in range(N + m):
            r = int(rows[s])
            t = times[s]
            if s < N:
                prefix = hist_t[: s + 1]
                act = int(hist_actions[a + s])
                pos = s
            else:
                prefix = hist_t + [req]
                act = n_action
                pos = N
            ri = len(set(prefix))
            earlier = [x for x in prefix if x < t]
            gap = (t - max(earlier)) if earlier else None
            bucket = 0 if gap is None else sum(1 for bk in bounds if bk <= gap)
            out["act"][r] = act
            out["pos"][r] = pos
            out["pe"][r] = min(pos, n_pos - 1)
            out["ri"][r] = ri
            out["ri_slot"][r] = min(ri - 1, n_ri - 1)
            out["gap"][r] = -1 if gap is None else gap
            out["rt"][r] = bucket
            out["tau"][r] = float(t - first)
    return out


# ----------------------------------------------------------------------------------------
# Embedding sum
# ----------------------------------------------------------------------------------------


def embed_sum(tables, hist_items, cand_items, idx, rows=None):
    """e_s = psi(x_s) + phi(a_s) + Omega_pe(p) + Omega_ri(ri) + Omega_rt(bucket), in fp64.

    [GR-zh] section 1.4.2, the five-term input representation (and section 1.4.1 for the
    item + action token and the mask-action row for candidates).  ``tables`` maps
    item/action/pos/ri/rt to float arrays [rows, d]; ``idx`` is ``token_indices``' output.
    """
    T_h = len(hist_items)
    T = len(idx["act"])
    rows = np.arange(T) if rows is None else np.asarray(rows)
    items = np.concatenate([np.asarray(hist_items, np.int64), np.asarray(cand_items, np.int64)])
    f = lambda name, ids: np.asarray(tables[name][ids], np.float64)
    x = (f("item", items[rows]) + f("action", idx["act"][rows]) + f("pos", idx["pe"][rows])
         + f("ri", idx["ri_slot"][rows]) + f("rt", idx["rt"][rows]))
    assert T_h <= T
    return x


def embed_bwd(dx, table_shapes, hist_items, cand_items, idx):
    """Gradients of the five tables: scatter-add of dx at each row's indices (the adjoint
    of ``embed_sum``)."""
    items = np.concatenate([np.asarray(hist_items, np.int64), np.asarray(cand_items, np.int64)])
    dx = np.asarray(dx, np.float64)
    grads = {k: np.zeros(s, np.float64) for k, s in table_shapes.items()}
    np.add.at(grads["item"], items, dx)
    np.add.at(grads["action"], idx["act"], dx)
    np.add.at(grads["pos"], idx["pe"], dx)
    np.add.at(grads["ri"], idx["ri_slot"], dx)
    np.add.at(grads["rt"], idx["rt"], dx)
    return grads


# ----------------------------------------------------------------------------------------
# Masked ALiBi attention
# ----------------------------------------------------------------------------------------


def attention_mask(N: int, m: int, history: str = "causal") -> np.ndarray:
    """allowed[i, j] for one user's sequence of N history actions then m candidates.

    History queries see history keys at or before them (causal mask); a candidate sees
    every history key and itself, never another candidate ([FR-en] section 7.2.1, the
    candidate mask; [GR-note], the worked example of one history item and two
    candidates; reading: the candidate's own key is visible, as when it is appended
    alone).  ``history="full"``: the variant in which every history query sees every
    history key ([GR-zh] section 1.3.1, the fully visible mask over the historical
    positions, as in T5); candidates are unchanged."""
    L = N + m
    allowed = np.zeros((L, L), dtype=bool)
    for i in range(L):
        if i < N:
            allowed[i, : (N if history == "full" else i + 1)] = True
        else:
            allowed[i, :N] = True
            allowed[i, i] = True
    return allowed


def time_bucket(gap, bounds):
    """#{k : bounds[k] <= gap} for non-negative integer gaps (the request-gap bucketing of
    the time embedding, [GR-zh] section 1.4.2), element-wise."""
    b = np.asarray(bounds, np.int64)
    g = np.asarray(gap, np.int64)
    return (b[None, :] <= g.reshape(-1)[:, None]).sum(axis=1).reshape(g.shape)


def _alibi_bias(pos, tau, sp, st, time_bounds=None):
    """-s_h |p_i - p_j| - s'_h |tau_i - tau_j| for one head ([GR-zh] section 1.4.2, the
    ALiBi score with position ids; time term as in [FR-en] section 7.2.2 with raw
    seconds).  With ``time_bounds`` the time term is -s'_h bucket(|tau_i - tau_j|): the
    page's -m_t bucket(t_i - t_j), reading: its bucket is the request-gap bucketing, on the
    absolute difference (for causal pairs t_i >= t_j, so the same as the page's)."""
    pos = np.asarray(pos, np.float64)
    tau = np.asarray(tau, np.float64)
    dt = np.abs(tau[:, None] - tau[None, :])
    if time_bounds is not None:
        dt = time_bucket(np.rint(dt).astype(np.int64), time_bounds).astype(np.float64)
    return -sp * np.abs(pos[:, None] - pos[None, :]) - st * dt


def attn_fwd_user(q, k, v, pos, tau, slopes_pos, slopes_time, N, m, history="causal", time_bounds=None):
    """One user's attention.  q, k, v: [L, H, dh] with L = N + m.

    score_ij = q_i . k_j / sqrt(dh) - s_h |p_i - p_j| - s'_h |tau_i - tau_j| on allowed
    pairs ([GR-zh] section 1.4.2, ALiBi score, d = head dimension); softmax over allowed
    keys; O = P V.  Returns (O [L, H, dh], lse [L, H]) with lse = log sum_j exp(score_ij).
    ``history`` and ``time_bounds``: the variants of ``attention_mask`` and ``_alibi_bias``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, H, dh = q.shape
    allowed = attention_mask(N, m, history)
    o = np.zeros_like(q)
    lse = np.zeros((L, H))
    for h in range(H):
        s = q[:, h, :] @ k[:, h, :].T / math.sqrt(dh)
        s = s + _alibi_bias(pos, tau, slopes_pos[h], slopes_time[h], time_bounds)
        s = np.where(allowed, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - mx), 0.0)
        z = e.sum(axis=1, keepdims=True)
        p = e / z
        o[:, h, :] = p @ v[:, h, :]
        lse[:, h] = mx[:, 0] + np.log(z[:, 0])
    return o, lse


def attn_fwd(q, k, v, hist_offsets, m, pos, tau, slopes_pos, slopes_time, users=None, history="causal",
             time_bounds=None):
    """Batch attention over jagged users; q/k/v [T, H, dh] in the shared row layout."""
    q = np.asarray(q, np.float64)
    B = len(hist_offsets) - 1
    o = np.zeros_like(q)
    lse = np.zeros(q.shape[:2])
    for u in (range(B) if users is None else users):
        rows = user_rows(hist_offsets, m, u)
        N = int(hist_offsets[u + 1] - hist_offsets[u])
        ou, lu = attn_fwd_user(q[rows], np.asarray(k)[rows], np.asarray(v)[rows], pos[rows],
                               tau[rows], slopes_pos, slopes_time, N, m, history, time_bounds)
        o[rows] = ou
        lse[rows] = lu
    return o, lse


def attn_bwd_user(q, k, v, do, pos, tau, slopes_pos, slopes_time, N, m, history="causal", time_bounds=None):
    """Gradients of one user's attention (the biases are constants: ALiBi has no
    parameters and needs no gradient, [GR-zh] section 1.4.2).

    With P the masked softmax: dV = P^T dO; dP = dO V^T; dS = P (dP - rowsum(P dP));
    dQ = dS K / sqrt(dh); dK = dS^T Q / sqrt(dh)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    L, H, dh = q.shape
    allowed = attention_mask(N, m, history)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(H):
        s = q[:, h, :] @ k[:, h, :].T / math.sqrt(dh)
        s = s + _alibi_bias(pos, tau, slopes_pos[h], slopes_time[h], time_bounds)
        s = np.where(allowed, s, -np.inf)
        e = np.where(allowed, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
        p = e / e.sum(axis=1, keepdims=True)
        dv[:, h, :] = p.T @ do[:, h, :]
        dp = do[:, h, :] @ v[:, h, :].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[:, h, :] = ds @ k[:, h, :] / math.sqrt(dh)
        dk[:, h, :] = ds.T @ q[:, h, :] / math.sqrt(dh)
    return dq, dk, dv


def attn_bwd(q, k, v, do, hist_offsets, m, pos, tau, slopes_pos, slopes_time, users=None, history="causal",
             time_bounds=None):
    q = np.asarray(q, np.float64)
    B = len(hist_offsets) - 1
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for u in (range(B) if users is None else users):
        rows = user_rows(hist_offsets, m, u)
        N = int(hist_offsets[u + 1] - hist_offsets[u])
        a, b, c = attn_bwd_user(q[rows], np.asarray(k)[rows], np.asarray(v)[rows],
                                np.asarray(do)[rows], pos[rows], tau[rows], slopes_pos,
                                slopes_time, N, m, history, time_bounds)
        dq[rows], dk[rows], dv[rows] = a, b, c
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Transformer block pieces.  The pages describe the backbone only as HSTU-derived blocks
# ([GR-zh] section 1.3 setup: 3 blocks, 8 heads, hidden 768).  Reading: pre-RMSNorm
# blocks with bias-free projections, residuals and a non-gated SiLU FFN; the
# single-layer inference form is embed -> QKV -> attention -> output projection.
# ----------------------------------------------------------------------------------------


def rmsnorm(x, g, eps=RMS_EPS):
    """y = x / sqrt(mean(x^2) + eps) * g, per row."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x * r * np.asarray(g, np.float64)


def rmsnorm_bwd(x, g, dy, eps=RMS_EPS):
    """Returns (dx, dg) for y = rmsnorm(x, g)."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    dy = np.asarray(dy, np.float64)
    d = x.shape[-1]
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    gdy = g * dy
    dx = r * gdy - (r ** 3) * x * (gdy * x).sum(axis=-1, keepdims=True) / d
    dg = (dy * x * r).sum(axis=0)
    return dx, dg


def silu(a):
    a = np.asarray(a, np.float64)
    return a / (1.0 + np.exp(-a))


def silu_bwd(a, dy):
    a = np.asarray(a, np.float64)
    sg = 1.0 / (1.0 + np.exp(-a))
    return np.asarray(dy, np.float64) * sg * (1.0 + a * (1.0 - sg))


def _split_heads(t, H):
    return t.reshape(t.shape[0], H, -1)


def round_bf16(x):
    """Storage rounding to bfloat16: the value is rounded to float32, then to the nearest
    bfloat16 (float32's sign and 8-bit exponent, the top 7 of its 23 fraction bits), ties
    to the even fraction; returned as float64.  Not part of the method: it models a
    tensor held in bf16 between two operations (see ``store`` below)."""
    b = np.asarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    kept = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (kept << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _identity(t):
    return t


def _stored(store, name):
    """The storage model of one named tensor: ``store`` is None (exact), one callable for
    every tensor, or a dict from tensor name to callable (names missing from it are exact)."""
    if store is None:
        return _identity
    if callable(store):
        return store
    return store.get(name, _identity)


def layer_fwd(x, lw, block, H, geom, store=None):
    """One block.  ``lw``: dict with wqkv [3d, d], wo [d, d], and for the pre-norm block
    w1 [f d, d], w2 [d, f d], g1, g2.  ``geom``: dict with hist_offsets, m, pos, tau,
    slopes_pos, slopes_time.  Returns (y, cache).

    ``store`` (default: none) is applied to every intermediate tensor that an
    implementation holds in memory between two operations: the normalised input "z",
    "qkv", the attention output "o", the residual sum "x1", the FFN hidden activation "hdn"
    (and "z2", its normalised input) and the output "y".  With ``store=round_bf16`` this is
    the same computation with those tensors kept in bf16, which measures the error that bf16
    storage alone brings; a dict {name: callable} models tensors kept in different types
    (say the residual sums in f32 and the rest in bf16)."""
    S = lambda name, t: _stored(store, name)(t)
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    wqkv = np.asarray(lw["wqkv"], np.float64)
    wo = np.asarray(lw["wo"], np.float64)
    cache = {"x": x}
    z = S("z", rmsnorm(x, lw["g1"])) if block == "prenorm" else x
    qkv = S("qkv", z @ wqkv.T)
    q, k, v = (_split_heads(qkv[:, i * d:(i + 1) * d], H) for i in range(3))
    o, _ = attn_fwd(q, k, v, geom["hist_offsets"], geom["m"], geom["pos"], geom["tau"],
                    geom["slopes_pos"], geom["slopes_time"], history=geom.get("history", "causal"),
                    time_bounds=geom.get("time_bounds"))
    o2 = S("o", o.reshape(o.shape[0], d))
    attn_out = o2 @ wo.T
    cache.update(z=z, q=q, k=k, v=v, o=o2)
    if block == "attn_only":
        return S("y", attn_out), cache
    x1 = S("x1", x + attn_out)
    z2 = S("z2", rmsnorm(x1, lw["g2"]))
    a = z2 @ np.asarray(lw["w1"], np.float64).T
    hdn = S("hdn", silu(a))
    y = S("y", x1 + hdn @ np.asarray(lw["w2"], np.float64).T)
    cache.update(x1=x1, z2=z2, a=a, hdn=hdn)
    return y, cache


def layer_bwd(dy, lw, block, H, geom, cache):
    """Backward of ``layer_fwd``.  Returns (dx, grads dict)."""
    dy = np.asarray(dy, np.float64)
    d = dy.shape[1]
    wqkv = np.asarray(lw["wqkv"], np.float64)
    wo = np.asarray(lw["wo"], np.float64)
    grads = {}
    if block == "attn_only":
        d_attn_out = dy
        dx_res = 0.0
    else:
        w1 = np.asarray(lw["w1"], np.float64)
        w2 = np.asarray(lw["w2"], np.float64)
        grads["w2"] = dy.T @ cache["hdn"]
        dhdn = dy @ w2
        da = silu_bwd(cache["a"], dhdn)
        grads["w1"] = da.T @ cache["z2"]
        dz2 = da @ w1
        dx1_norm, grads["g2"] = rmsnorm_bwd(cache["x1"], lw["g2"], dz2)
        dx1 = dy + dx1_norm
        d_attn_out = dx1
        dx_res = dx1
    grads["wo"] = d_attn_out.T @ cache["o"]
    do = (d_attn_out @ wo).reshape(-1, H, d // H)
    dq, dk, dv = attn_bwd(cache["q"], cache["k"], cache["v"], do, geom["hist_offsets"],
                          geom["m"], geom["pos"], geom["tau"], geom["slopes_pos"],
                          geom["slopes_time"], history=geom.get("history", "causal"),
                          time_bounds=geom.get("time_bounds"))
    dqkv = np.concatenate([t.reshape(-1, d) for t in (dq, dk, dv)], axis=1)
    grads["wqkv"] = dqkv.T @ cache["z"]
    dz = dqkv @ wqkv
    if block == "attn_only":
        return dz, grads
    dx_norm, grads["g1"] = rmsnorm_bwd(cache["x"], lw["g1"], dz)
    return dx_res + dx_norm, grads


def head_fwd(x_cand, g_final, w_head, b_head):
    """Per-candidate action logits: RMSNorm, then a [n_tasks, d] projection plus bias
    (a set of predefined tasks per candidate, [GR-zh] section 1.2; reading: one linear
    head with 4 logits)."""
    z = rmsnorm(x_cand, g_final)
    return z @ np.asarray(w_head, np.float64).T + np.asarray(b_head, np.float64)


def head_bwd(dlogits, x_cand, g_final, w_head):
    dlogits = np.asarray(dlogits, np.float64)
    z = rmsnorm(x_cand, g_final)
    grads = {"w_head": dlogits.T @ z, "b_head": dlogits.sum(axis=0)}
    dz = dlogits @ np.asarray(w_head, np.float64)
    dx, grads["g_final"] = rmsnorm_bwd(x_cand, g_final, dz)
    return dx, grads


def bce_loss(logits, labels):
    """Mean sigmoid binary cross-entropy over every candidate and task; loss is taken at
    candidate positions only ([GR-zh] section 1.3.1).  Reading: mean reduction."""
    z = np.asarray(logits, np.float64)
    y = np.asarray(labels, np.float64)
    softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    return float((softplus - y * z).mean())


def bce_loss_bwd(logits, labels):
    z = np.asarray(logits, np.float64)
    y = np.asarray(labels, np.float64)
    return (1.0 / (1.0 + np.exp(-z)) - y) / z.size


def _loss_rows(geom, n_rows, loss_rows):
    """The rows that carry a loss: the candidate rows [T_h, T) by default ([GR-zh] section
    1.3.1, loss at candidate positions only), else the given row indices (the section's
    ablation that also takes the loss at some history positions)."""
    if loss_rows is None:
        return np.arange(int(geom["hist_offsets"][-1]), n_rows)
    return np.asarray(loss_rows, np.int64)


def model_fwd(x0, layers, block, H, geom, head=None, store=None, loss_rows=None):
    """Embedded rows -> stacked blocks -> (optional) head at the loss rows (candidate rows
    unless ``loss_rows`` lists others).  Returns (x_final, logits or None, caches).
    ``store``: as in ``layer_fwd``, also applied to the embedded rows ("x0")."""
    x = _stored(store, "x0")(np.asarray(x0, np.float64))
    caches = []
    for lw in layers:
        x, c = layer_fwd(x, lw, block, H, geom, store)
        caches.append(c)
    logits = None
    if head is not None:
        rows = _loss_rows(geom, x.shape[0], loss_rows)
        logits = head_fwd(x[rows], head["g_final"], head["w_head"], head["b_head"])
    return x, logits, caches


def model_bwd(dlogits, x_final, layers, block, H, geom, caches, head, loss_rows=None):
    """Backward through the head and the blocks.  Returns (dx0, per-layer grads, head grads)."""
    rows = _loss_rows(geom, np.asarray(x_final).shape[0], loss_rows)
    dx = np.zeros_like(np.asarray(x_final, np.float64))
    dxc, hgrads = head_bwd(dlogits, x_final[rows], head["g_final"], head["w_head"])
    np.add.at(dx, rows, dxc)
    lgrads = [None] * len(layers)
    for li in range(len(layers) - 1, -1, -1):
        dx, lgrads[li] = layer_bwd(dx, layers[li], block, H, geom, caches[li])
    return dx, lgrads, hgrads


# ----------------------------------------------------------------------------------------
# HSTU-style interleaved sequence with a learned relative attention bias (the comparison
# the pages draw: [FR-en] section 7.2.1 interleaving, section 7.2.2 relative attention
# bias, an N x N matrix read in the forward pass).
# ----------------------------------------------------------------------------------------


def hstu_sequence(N: int, m: int):
    """Interleaved slots [x_1, a_1, ..., x_N, a_N, c_1..c_m] of length 2N + m.  Returns
    (kind, src, pos) where kind is 0 item token / 1 action token / 2 candidate,
    src the history index (or candidate index), pos the position id (candidates share 2N).
    Reading: candidate tokens carry the candidate item."""
    L = 2 * N + m
    kind = np.zeros(L, np.int64)
    src = np.zeros(L, np.int64)
    pos = np.zeros(L, np.int64)
    for i in range(N):
        kind[2 * i], src[2 * i], pos[2 * i] = 0, i, 2 * i
        kind[2 * i + 1], src[2 * i + 1], pos[2 * i + 1] = 1, i, 2 * i + 1
    for c in range(m):
        kind[2 * N + c], src[2 * N + c], pos[2 * N + c] = 2, c, 2 * N
    return kind, src, pos


def hstu_rab(pos, t, pos_table, time_table, time_bounds):
    """Learned relative bias rab_ij = pos_table[min(|p_i - p_j|, P-1)] +
    time_table[#{k : b_k <= |t_i - t_j|}] (reading of [FR-en] section 7.2.2: a learned
    function of position and time difference)."""
    pos = np.asarray(pos, np.int64)
    t = np.asarray(t, np.int64)
    P = len(pos_table)
    dp = np.minimum(np.abs(pos[:, None] - pos[None, :]), P - 1)
    dt = np.abs(t[:, None] - t[None, :])
    bt = np.zeros_like(dt)
    for bk in time_bounds:
        bt += (dt >= int(bk)).astype(np.int64)
    return np.asarray(pos_table, np.float64)[dp] + np.asarray(time_table, np.float64)[bt]


def hstu_attn_fwd_user(q, k, v, rab, N, m):
    """Softmax attention over the interleaved sequence with bias ``rab`` [L, L] (one matrix
    shared by the heads); history slots causal, candidates see all 2N history slots and
    themselves.  q/k/v [L, H, dh].  Returns (O [L, H, dh], lse [L, H])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, H, dh = q.shape
    allowed = attention_mask(2 * N, m)
    o = np.zeros_like(q)
    lse = np.zeros((L, H))
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(dh) + np.asarray(rab, np.float64)
        s = np.where(allowed, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - mx), 0.0)
        z = e.sum(axis=1, keepdims=True)
        o[:, h] = (e / z) @ v[:, h]
        lse[:, h] = mx[:, 0] + np.log(z[:, 0])
    return o, lse


def hstu_times(hist_ts, req_t, N, m):
    """Times of the interleaved slots: both tokens of history action i carry t_i, the
    candidates the request time (reading: an action happens at its item's time)."""
    t = np.empty(2 * N + m, np.int64)
    t[0:2 * N:2] = hist_ts[:N]
    t[1:2 * N:2] = hist_ts[:N]
    t[2 * N:] = req_t
    return t
