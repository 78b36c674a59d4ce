"""The seeded input generators: shapes and the structural properties the pages give."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        # exact ties between two bf16 values (round half to even)
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny_fp32", "infer_1layer_bf16", "train2_bf16"])
def test_batch_structure(name):
    cfg = synth.make_config(name)
    b = synth.make_batch(cfg, B=min(cfg.B, 24))
    n = b.lengths
    assert b.hist_offsets[0] == 0 and np.all(n >= cfg.hist_min) and np.all(n <= cfg.hist_max)
    assert len(b.hist_items) == len(b.hist_actions) == len(b.hist_ts) == b.total_hist
    assert len(b.cand_items) == b.B * cfg.m
    assert b.hist_items.min() >= 0 and b.hist_items.max() < cfg.n_item
    assert b.hist_actions.min() >= 0 and b.hist_actions.max() < cfg.n_action
    for u in range(b.B):
        ts = b.hist_ts[b.hist_offsets[u]:b.hist_offsets[u + 1]]
        assert np.all(np.diff(ts) >= 0)
        assert b.req_ts[u] > ts[-1]
        # requests are runs of 1..4 items sharing one timestamp
        _, counts = np.unique(ts, return_counts=True)
        assert counts.max() <= 4 or len(ts) < 1


def test_first_users_do_not_depend_on_batch_size():
    cfg = synth.make_config("infer_1layer_bf16")
    a = synth.make_batch(cfg, B=3)
    b = synth.make_batch(cfg, B=7).subset([0, 1, 2])
    for f in ("hist_offsets", "hist_items", "hist_actions", "hist_ts", "cand_items", "req_ts"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_zipf_ids_are_frequency_ordered():
    cfg = synth.make_config("infer_1layer_bf16")
    b = synth.make_batch(cfg, B=64)
    ids = np.concatenate([b.hist_items, b.cand_items])
    # Zipf(1.1) over 1e6: the top 100 ids take roughly half of the draws
    frac_top100 = np.mean(ids < 100)
    assert 0.4 < frac_top100 < 0.65
    assert np.mean(ids == 0) > np.mean(ids == 1) > np.mean(ids == 5)


def test_rt_boundaries_log_spaced_integers():
    b = synth.rt_boundaries(64)
    assert len(b) == 63 and b[0] == 1 and b[-1] == 2 ** 24
    assert np.all(np.diff(b) >= 1)
