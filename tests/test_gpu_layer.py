"""GPU parity of the block forward (embed -> QKV -> attention -> output projection [-> FFN])
and the action head, through the same GenRank model wrapper the benchmark drives.

Bars: f32 <= 1e-5 absolute; bf16 logits (unit-scale) <= 2e-2 absolute (the pre-norm stacks keep
their residual stream in f32, the projections' operands in bf16); bf16 hidden states
(scale ~1e-3 with N(0, 0.02) weights) by ``bf16_close``: norm-wise <= 1e-2 and max error
<= 2e-2 of the tensor's largest magnitude."""
import numpy as np
import pytest
import torch

import oracle
import synth
from common import oracle_geom, oracle_head, oracle_indices, oracle_layers, oracle_tables
from gpu_common import (DEV, DeviceInputs, GenRank, bf16_close, custom_batch, f32_resid_store, gpu_slopes, say,
                        tables_for, to_numpy, unit_close)

pytestmark = pytest.mark.gpu


def _oracle_forward(cfg, batch, tables, weights, store=None):
    idx = oracle_indices(cfg, batch, tables)
    x = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    geom = oracle_geom(cfg, batch, idx)
    head = oracle_head(weights) if cfg.block == "prenorm" else None
    y, logits, _ = oracle.model_fwd(x, oracle_layers(weights), cfg.block, cfg.H, geom, head, store=store)
    return y, logits


def _gpu_forward(cfg, batch, tables, weights):
    sp, st = gpu_slopes(cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, DEV)
    inp = DeviceInputs(batch, DEV)
    y, logits = model.forward(inp)
    torch.cuda.synchronize()
    return to_numpy(y), (logits.cpu().numpy().astype(np.float64) if logits is not None else None)


@pytest.mark.parametrize("block", ["attn_only", "prenorm"])
def test_layer_f32_tiny(block):
    say(f"layer: f32 tiny {block}")
    cfg = synth.make_config("tiny_fp32", block=block, layers=2 if block == "prenorm" else 1)
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    gy, gl = _gpu_forward(cfg, batch, tables, weights)
    wy, wl = _oracle_forward(cfg, batch, tables, weights)
    assert np.abs(gy - wy).max() <= 1e-5
    if wl is not None:
        assert np.abs(gl - wl).max() <= 1e-5


def test_layer_f32_jagged_prenorm():
    say("layer: f32 jagged prenorm")
    cfg = synth.make_config("tiny_fp32", block="prenorm", layers=2, m=3, d=64, H=4,
                            slopes_pos=(0.5, 0.25, 0.125, 0.0625), slopes_time=(0.1, 0.05, 0.02, 0.01))
    batch = custom_batch(cfg, [0, 5, 70, 33], seed=2)
    tables, weights = synth.make_tables(cfg), synth.make_weights(cfg)
    gy, gl = _gpu_forward(cfg, batch, tables, weights)
    wy, wl = _oracle_forward(cfg, batch, tables, weights)
    assert np.abs(gy - wy).max() <= 1e-5
    assert np.abs(gl - wl).max() <= 1e-5


def test_layer_bf16_infer_subset():
    """infer_1layer_bf16 (embed -> QKV -> attention -> Wo, no norm / residual) on 12 users."""
    say("layer: bf16 infer subset")
    cfg = synth.make_config("infer_1layer_bf16")
    batch = synth.make_batch(cfg, B=12)
    tables, weights = tables_for("infer_1layer_bf16"), synth.make_weights(cfg)
    gy, _ = _gpu_forward(cfg, batch, tables, weights)
    wy, _ = _oracle_forward(cfg, batch, tables, weights)
    bf16_close(gy, wy, "y")


def test_stack_bf16_small_batch():
    """stack4_bf16 shapes (4 pre-norm layers, d = 512, 8 heads, FFN 4x, head of 4 logits)
    on 3 users with jagged lengths, with the stack's f32 residual stream: logits within
    2e-2 of the exact oracle.  The error of the same computation with the stack's storage
    (bf16 operands, f32 residual rows) and exact arithmetic otherwise is printed beside it,
    and the kernels' rms error must stay within 1.25x of it."""
    say("layer: bf16 stack4 small batch")
    cfg = synth.make_config("stack4_bf16", m=40)
    batch = custom_batch(cfg, [480, 123, 7], seed=4)
    tables = tables_for("stack4_bf16")
    weights = synth.make_weights(cfg)
    gy, gl = _gpu_forward(cfg, batch, tables, weights)
    wy, wl = _oracle_forward(cfg, batch, tables, weights)
    _, sl = _oracle_forward(cfg, batch, tables, weights, store=f32_resid_store())
    assert np.std(wl) > 0.3  # the logits are unit-scale
    rms = lambda e: float(np.sqrt(np.mean(np.square(e))))
    e_gpu, e_store = gl - wl, sl - wl
    say(f"  logits: gpu rms {rms(e_gpu):.4f} max {np.abs(e_gpu).max():.4f}; "
        f"storage alone rms {rms(e_store):.4f} max {np.abs(e_store).max():.4f}")
    assert rms(e_gpu) <= 1.25 * rms(e_store), (rms(e_gpu), rms(e_store))
    unit_close(gl, wl, "logits", tol=2e-2)
    bf16_close(gy, wy, "final hidden state")


def test_layer_bf16_full_size_sampled():
    """The full infer_1layer_bf16 batch (256 users) as the benchmark runs it; 4 users checked
    against the oracle (users are independent, so a sub-batch is exact)."""
    say("layer: bf16 full infer batch, sampled users")
    cfg = synth.make_config("infer_1layer_bf16")
    batch = synth.make_batch(cfg)
    tables, weights = tables_for("infer_1layer_bf16"), synth.make_weights(cfg)
    gy, _ = _gpu_forward(cfg, batch, tables, weights)
    assert np.isfinite(gy).all()
    users = [3, 64, 190, 255]
    sub = batch.subset(users)
    wy, _ = _oracle_forward(cfg.replace(B=len(users)), sub, tables, weights)
    rows = np.concatenate([oracle.user_rows(batch.hist_offsets, cfg.m, u) for u in users])
    sub_rows = np.concatenate([oracle.user_rows(sub.hist_offsets, cfg.m, i) for i in range(len(users))])
    bf16_close(gy[rows], wy[sub_rows], "y (sampled users)")


def test_stack_bf16_full_size_sampled():
    """The full 4-layer stack batch (512 users, 480 history actions and 256 candidates each:
    376,832 rows, d = 512) in the launches the benchmark runs (the 256 x 256-tile
    projections included); 3 users' logits and final hidden states checked against the
    oracle on those users alone (users are independent).  Logit bars as for the small
    stack batch: max error 2e-2, rms within 1.25x of the storage-only error."""
    say("layer: bf16 stack4 full batch, sampled users")
    cfg = synth.make_config("stack4_bf16")
    batch = synth.make_batch(cfg)
    tables, weights = tables_for("stack4_bf16"), synth.make_weights(cfg)
    sp, st = gpu_slopes(cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, DEV)
    inp = DeviceInputs(batch, DEV)
    y, logits = model.forward(inp)
    users = [0, 257, 511]
    rows = np.concatenate([oracle.user_rows(batch.hist_offsets, cfg.m, u) for u in users])
    gy = to_numpy(y[torch.as_tensor(rows, device=DEV)])
    gl = logits.view(batch.B, cfg.m, -1)[torch.as_tensor(users, device=DEV)].reshape(-1, logits.shape[1])
    gl = gl.cpu().numpy().astype(np.float64)
    finite = bool(torch.isfinite(logits).all()) and bool(torch.isfinite(y).all())
    del y, logits, model
    torch.cuda.synchronize()
    assert finite
    sub = batch.subset(users)
    c = cfg.replace(B=len(users))
    wy, wl = _oracle_forward(c, sub, tables, weights)
    _, sl = _oracle_forward(c, sub, tables, weights, store=f32_resid_store())
    rms = lambda e: float(np.sqrt(np.mean(np.square(e))))
    e_gpu, e_store = gl - wl, sl - wl
    say(f"  logits: gpu rms {rms(e_gpu):.4f} max {np.abs(e_gpu).max():.4f}; "
        f"storage alone rms {rms(e_store):.4f} max {np.abs(e_store).max():.4f}")
    assert rms(e_gpu) <= 1.25 * rms(e_store), (rms(e_gpu), rms(e_store))
    unit_close(gl, wl, "logits", tol=2e-2)
    sub_rows = np.concatenate([oracle.user_rows(sub.hist_offsets, cfg.m, i) for i in range(len(users))])
    bf16_close(gy, wy[sub_rows], "final hidden state (sampled users)")
