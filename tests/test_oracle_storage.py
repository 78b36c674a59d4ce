"""The oracle's bf16 storage model (``round_bf16`` and the ``store`` hook of the forward),
pinned to the bfloat16 format's definition: 8 significant bits, float32's exponent range,
round to nearest with ties to even.  No GPU."""
import math

import numpy as np

import oracle
import synth
from common import oracle_geom, oracle_head, oracle_indices, oracle_layers, oracle_tables


def _round_frexp(x):
    """Independent definition: scale the significand to 8 bits and round half to even
    (Python's round does ties-to-even)."""
    if x == 0.0:
        return 0.0
    m, e = math.frexp(float(np.float32(x)))  # x = m * 2**e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)


def test_round_bf16_fixed_points_and_ties():
    cases = {
        1.0: 1.0, -2.5: -2.5, 2.0 ** -7: 2.0 ** -7, 3.0: 3.0, 1 + 2.0 ** -7: 1 + 2.0 ** -7,
        1 + 2.0 ** -8: 1.0,                    # tie, even neighbour is 1.0
        1 + 3 * 2.0 ** -8: 1 + 2.0 ** -6,      # tie, even neighbour is the upper one
        1 + 2.0 ** -8 + 2.0 ** -12: 1 + 2.0 ** -7,
        -(1 + 2.0 ** -8 + 2.0 ** -12): -(1 + 2.0 ** -7),
        0.0: 0.0,
    }
    got = oracle.round_bf16(np.array(list(cases)))
    assert np.array_equal(got, np.array(list(cases.values())))


def test_round_bf16_matches_frexp_definition():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        rng.uniform(-1, 1, 1000)])
    got = oracle.round_bf16(x)
    want = np.array([_round_frexp(v) for v in x])
    assert np.array_equal(got, want)
    # representable: the low 16 bits of the float32 pattern are zero
    assert not np.any(got.astype(np.float32).view(np.uint32) & 0xFFFF)
    # unit roundoff of an 8-bit significand
    assert np.all(np.abs(got - x) <= 2.0 ** -8 * np.abs(x) * (1 + 1e-6))
    # monotone
    xs = np.sort(x)
    assert np.all(np.diff(oracle.round_bf16(xs)) >= 0)


def test_store_hook():
    cfg = synth.make_config("tiny_fp32", block="prenorm", layers=2)
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    idx = oracle_indices(cfg, batch, tables)
    x0 = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    geom = oracle_geom(cfg, batch, idx)
    layers, head = oracle_layers(weights), oracle_head(weights)
    y, lg, _ = oracle.model_fwd(x0, layers, cfg.block, cfg.H, geom, head)
    y1, lg1, _ = oracle.model_fwd(x0, layers, cfg.block, cfg.H, geom, head, store=lambda t: t)
    assert np.array_equal(y, y1) and np.array_equal(lg, lg1)
    ys, lgs, caches = oracle.model_fwd(x0, layers, cfg.block, cfg.H, geom, head, store=oracle.round_bf16)
    # every stored tensor is representable in bf16
    for c in caches:
        for name in ("z", "o", "x1", "z2", "hdn"):
            assert not np.any(c[name].astype(np.float32).view(np.uint32) & 0xFFFF), name
    assert not np.any(ys.astype(np.float32).view(np.uint32) & 0xFFFF)
    # and the result moves by about bf16's resolution, not more
    rel = np.abs(ys - y).max() / np.abs(y).max()
    assert 0 < rel < 2.0 ** -4


def test_store_hook_by_name():
    """A dict storage model rounds only the named tensors: with the residual sums ("x0",
    "x1", "y") kept exact and every other stored tensor rounded to bf16, the residual
    tensors are untouched by rounding (the block output of the last layer is the exact sum
    of its stored inputs) while the operands are bf16."""
    cfg = synth.make_config("tiny_fp32", block="prenorm", layers=2)
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    idx = oracle_indices(cfg, batch, tables)
    x0 = oracle.embed_sum(oracle_tables(tables), batch.hist_items, batch.cand_items, idx)
    geom = oracle_geom(cfg, batch, idx)
    layers, head = oracle_layers(weights), oracle_head(weights)
    ops = {k: oracle.round_bf16 for k in ("z", "qkv", "o", "z2", "hdn")}
    y, _, caches = oracle.model_fwd(x0, layers, cfg.block, cfg.H, geom, head, store=ops)
    for c in caches:
        for name in ("z", "o", "z2", "hdn"):
            assert not np.any(c[name].astype(np.float32).view(np.uint32) & 0xFFFF), name
    # x0 is passed through unrounded
    assert np.array_equal(caches[0]["x"], x0)
    # y = x1 + hdn W2^T exactly (no rounding of the sum)
    last = caches[-1]
    want = last["x1"] + last["hdn"] @ np.asarray(layers[-1]["w2"], np.float64).T
    assert np.array_equal(y, want)
    # the name "y" alone rounds only the block outputs
    y2, _, c2 = oracle.model_fwd(x0, layers, cfg.block, cfg.H, geom, head, store={"y": oracle.round_bf16})
    assert not np.any(y2.astype(np.float32).view(np.uint32) & 0xFFFF)
    assert np.array_equal(c2[0]["x"], x0)
