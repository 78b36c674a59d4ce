"""Serving with cached history keys and values: a request's candidate rows against the
users' history K/V computed earlier.  History rows never depend on candidates (the mask:
history queries see earlier history keys only), so the cached path must reproduce the
candidate rows of the full forward exactly, on the same kernels: bit-identical outputs and
logits.  The full forward itself is held to the oracle in test_gpu_layer.py; here one user
is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from common import oracle_geom, oracle_indices, oracle_layers, oracle_slopes, oracle_tables
from gpu_common import (DEV, DeviceInputs, GenRank, batch_struct, custom_batch, gpu_slopes, random_qkv, say,
                        to_numpy, unit_close)
from generative_ranking_recommendation_amd import binding as B
from generative_ranking_recommendation_amd.device import stored_to_device

pytestmark = pytest.mark.gpu


# the full forward runs the LDS-resident pair kernel for histories up to 576 keys (the ring
# kernel beyond), the cached one the ring kernel: the candidate rows must agree bit for bit
@pytest.mark.parametrize("lengths,m", [
    ([64, 300, 480, 5, 0, 1], 32),
    ([129, 0, 200], 130),
    ([480, 480, 17], 256),           # the stack workload's top block
    ([600, 30], 200),                # a history past 576 keys: the ring kernel on both sides
])
# both outputs have row stride d + pad: pad 8 keeps the full forward's rows 16-byte aligned (the
# pair kernel's stores); with pad 4 it takes the ring kernel too
@pytest.mark.parametrize("pad", [8, 4])
def test_attn_fwd_cached_equals_full(lengths, m, pad):
    say(f"serving: cached attention {lengths} m={m} output pad {pad}")
    cfg = synth.make_config("train2_bf16", m=m)
    batch = custom_batch(cfg, lengths, seed=5)
    d, H = cfg.d, cfg.H
    T, Th = batch.total_rows, batch.total_hist
    st, _ = random_qkv(T, d, cfg.dtype, seed=51)
    inp = DeviceInputs(batch, DEV)
    bt = batch_struct(cfg, inp)
    qkv = stored_to_device(st, DEV)
    es = 2
    sl = B.HostSlopes(*gpu_slopes(cfg))
    o = torch.full((T, d + pad), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    p = qkv.data_ptr()
    B.genrank_attn_fwd(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, sl, p, p + d * es, p + 2 * d * es, 3 * d,
                       o, d + pad, lse)
    # history K/V as a separate cache [T_h, 2d]; candidate q/k/v rows as their own buffer
    kv = qkv[:Th, d:].contiguous()
    qc = qkv[Th:].contiguous()
    oc = torch.full((T - Th, d + pad), 7.0, dtype=torch.bfloat16, device=DEV)
    lc = torch.empty((T - Th, H), dtype=torch.float32, device=DEV)
    c, k = qc.data_ptr(), kv.data_ptr()
    B.genrank_attn_fwd_cached(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, sl, c, c + d * es, c + 2 * d * es,
                              3 * d, k, k + d * es, 2 * d, oc, d + pad, lc)
    torch.cuda.synchronize()
    assert torch.equal(oc[:, :d], o[Th:, :d]), "candidate outputs differ"
    assert torch.equal(lc, lse[Th:]), "candidate log-sum-exp differs"
    assert bool((oc[:, d:].float() == 7.0).all()) and bool((o[:, d:].float() == 7.0).all())


def _model(cfg, batch):
    sp, st = gpu_slopes(cfg)
    model = GenRank.from_host(cfg, synth.make_tables(cfg), synth.make_weights(cfg), sp, st, DEV)
    return model, DeviceInputs(batch, DEV)


@pytest.mark.parametrize("name,lengths,m", [
    ("infer_1layer_bf16", [0, 1, 63, 64, 65, 480, 300], 130),
    ("stack4_bf16", [480, 123, 7, 0], 40),
    ("stack4_bf16", [480, 480, 31], 256),
    ("train2_bf16", [64, 300, 480, 5], 32),
])
def test_score_equals_forward(name, lengths, m):
    say(f"serving: score vs forward {name} {lengths} m={m}")
    cfg = synth.make_config(name, m=m)
    batch = custom_batch(cfg, lengths, seed=9)
    model, inp = _model(cfg, batch)
    x_full, logits_full = model.forward(inp)
    caches = model.prefill(inp)
    x_c, logits_c = model.score(inp, caches)
    torch.cuda.synchronize()
    Th = inp.total_hist
    assert torch.equal(x_c, x_full[Th:]), "candidate rows differ"
    if logits_full is not None:
        assert torch.equal(logits_c, logits_full), "logits differ"


def test_score_single_layer_against_oracle():
    """The cached single-layer path against the oracle on the candidate rows (unit-scale
    q, k, v are not available here: the block output is held to the non-unit-scale bar)."""
    say("serving: single layer vs oracle")
    from gpu_common import bf16_close
    cfg = synth.make_config("infer_1layer_bf16", m=20)
    batch = custom_batch(cfg, [200, 0, 31], seed=3)
    tables, weights = synth.make_tables(cfg), synth.make_weights(cfg)
    sp, st = gpu_slopes(cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, DEV)
    inp = DeviceInputs(batch, DEV)
    x_c, _ = model.score(inp, model.prefill(inp))
    idx = oracle_indices(cfg, batch, tables)
    x0 = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    y, _, _ = oracle.model_fwd(x0, oracle_layers(weights), cfg.block, cfg.H, oracle_geom(cfg, batch, idx))
    bf16_close(to_numpy(x_c), y[batch.total_hist:], "candidate block output")


@pytest.mark.parametrize("name,lengths,m", [
    ("infer_1layer_bf16", [0, 1, 63, 64, 65, 480, 300], 130),
    ("stack4_bf16", [480, 123, 7, 0], 40),
])
def test_score_graph_replay(name, lengths, m):
    """Cached scoring captured once in a HIP graph (the entry points take the capturing
    stream; none of them allocates, synchronises or clears memory with a memset): each of
    several replays, with the program's own eager scoring and synchronisations between them,
    reproduces the eager rows and logits bit for bit."""
    say(f"serving: graph replay {name} {lengths} m={m}")
    cfg = synth.make_config(name, m=m)
    batch = custom_batch(cfg, lengths, seed=9)
    model, inp = _model(cfg, batch)
    caches = model.prefill(inp)
    x_ref, logits_ref = model.score(inp, caches)  # eager; also sets up every lazily made buffer
    torch.cuda.synchronize()
    x_ref = x_ref.clone()
    logits_ref = None if logits_ref is None else logits_ref.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        x_g, logits_g = model.score(inp, caches)
    for r in range(3):
        x_g.fill_(float("nan"))
        if logits_g is not None:
            logits_g.fill_(float("nan"))
        x_e, _ = model.score(inp, caches)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(x_e, x_ref)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x_g, x_ref), f"replay {r}: rows differ"
        if logits_ref is not None:
            assert torch.equal(logits_g, logits_ref), f"replay {r}: logits differ"
