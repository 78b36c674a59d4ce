"""Pins for the oracle's index derivation and embedding sum (no GPU).

Each check is fixed by the pages or by arithmetic independent of the oracle's code:
printed examples (tests/golden), hand-worked vectors, and an alternative closed form of
the set definitions that holds for sorted timestamps."""
import json
import os

import numpy as np

import oracle
import synth
from common import oracle_indices, oracle_tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _one_user(ts, req, m=1, acts=None, n_action=8, n_pos=16, n_ri=8, bounds=(1, 5, 30, 100)):
    offs = np.array([0, len(ts)], np.int64)
    acts = np.zeros(len(ts), np.int64) if acts is None else np.asarray(acts)
    return oracle.token_indices(offs, acts, np.asarray(ts, np.int64), np.array([req]), m,
                                n_action, n_pos, n_ri, np.asarray(bounds, np.int64))


def test_request_index_and_gap_hand_vector():
    g = _load("request_index_hand_vector.json")
    idx = _one_user(g["hist_ts"], g["req_ts"], m=1)
    N = len(g["hist_ts"])
    assert idx["ri"][:N].tolist() == g["history_request_index"]
    gaps = [None if x < 0 else int(x) for x in idx["gap"][:N]]
    assert gaps == g["history_gap"]
    assert idx["ri"][N] == g["candidate_request_index"]
    assert idx["gap"][N] == g["candidate_gap"]


def test_candidates_share_one_position():
    g = _load("shared_candidate_position.json")
    N, m = g["history_length"], g["candidates"]
    ts = np.arange(N) * 10
    idx = _one_user(ts, ts[-1] + 5, m=m, n_pos=512, n_ri=512)
    assert idx["pos"][:N].tolist() == list(range(N))
    expected0 = g["candidate_position_one_based"] - 1
    assert idx["pos"][N:].tolist() == [expected0] * m
    assert idx["act"][N:].tolist() == [8] * m  # mask-action row


def test_sorted_closed_form_random():
    """For non-decreasing timestamps the set definitions reduce to: request index = 1 +
    number of timestamp changes so far; gap = t_s - (previous distinct timestamp)."""
    cfg = synth.make_config("infer_1layer_bf16")
    b = synth.make_batch(cfg, B=5)
    bounds = synth.rt_boundaries(cfg.n_rt)
    idx = oracle.token_indices(b.hist_offsets, b.hist_actions, b.hist_ts, b.req_ts, b.m,
                               cfg.n_action, cfg.n_pos, cfg.n_ri, bounds)
    T_h = b.total_hist
    for u in range(b.B):
        a, e = b.hist_offsets[u], b.hist_offsets[u + 1]
        ts = b.hist_ts[a:e]
        change = np.concatenate([[0], (np.diff(ts) != 0).astype(np.int64)])
        ri = 1 + np.cumsum(change)
        assert np.array_equal(idx["ri"][a:e], ri)
        distinct = np.unique(ts)
        for s in range(len(ts)):
            k = np.searchsorted(distinct, ts[s])
            gap = -1 if k == 0 else ts[s] - distinct[k - 1]
            assert idx["gap"][a + s] == gap
            want_bucket = 0 if gap < 0 else int(np.searchsorted(bounds, gap, side="right"))
            assert idx["rt"][a + s] == want_bucket
        cand = T_h + u * b.m + np.arange(b.m)
        assert np.all(idx["ri"][cand] == ri[-1] + 1)
        assert np.all(idx["gap"][cand] == b.req_ts[u] - ts[-1])
        assert np.all(idx["pos"][cand] == e - a)
        assert np.all(idx["tau"][cand] == float(b.req_ts[u] - ts[0]))
        assert np.array_equal(idx["tau"][a:e], (ts - ts[0]).astype(np.float64))


def test_unsorted_timestamps_follow_set_definitions():
    # ts [30, 10, 20]: distinct counts 1, 2, 3; "earlier" sets {} , {} , {10}
    idx = _one_user([30, 10, 20], 40, m=1)
    assert idx["ri"][:3].tolist() == [1, 2, 3]
    assert idx["gap"][:3].tolist() == [-1, -1, 10]
    assert idx["ri"][3] == 4 and idx["gap"][3] == 10  # max{t < 40} = 30


def test_bucket_edges_and_clamps():
    # boundaries (1, 5, 30, 100): gap 5 is in bucket 2 (edges count), gap 4 in bucket 1
    idx = _one_user([0, 4, 9, 39, 139, 1000], 1001, m=2, n_pos=3, n_ri=2)
    assert idx["gap"][:6].tolist() == [-1, 4, 5, 30, 100, 861]
    assert idx["rt"][:6].tolist() == [0, 1, 2, 3, 4, 4]
    assert idx["pe"].tolist() == [0, 1, 2, 2, 2, 2, 2, 2]          # clamped to n_pos - 1
    assert idx["ri_slot"].tolist() == [0, 1, 1, 1, 1, 1, 1, 1]     # clamped to n_ri - 1
    assert idx["pos"].tolist() == [0, 1, 2, 3, 4, 5, 6, 6]          # raw ids stay unclamped


def test_empty_history_user():
    idx = _one_user([], 500, m=3)
    assert idx["pos"].tolist() == [0, 0, 0]
    assert idx["ri"].tolist() == [1, 1, 1]
    assert idx["rt"].tolist() == [0, 0, 0]
    assert idx["tau"].tolist() == [0.0, 0.0, 0.0]


def test_embed_sum_picks_the_right_rows():
    """Tables whose rows encode their own index: the sum reveals each table's row."""
    cfg = synth.make_config("tiny_fp32")
    b = synth.make_batch(cfg)
    tables = synth.make_tables(cfg)
    d = cfg.d
    enc = {}
    for t, name in enumerate(("item", "action", "pos", "ri", "rt")):
        rows = getattr(tables, name).shape[0]
        a = np.zeros((rows, d))
        a[:, t] = np.arange(rows)
        enc[name] = a
    idx = oracle_indices(cfg, b, tables)
    x = oracle.embed_sum(enc, b.hist_items, b.cand_items, idx)
    items = np.concatenate([b.hist_items, b.cand_items])
    assert np.array_equal(x[:, 0], items)
    assert np.array_equal(x[:, 1], idx["act"])
    assert np.array_equal(x[:, 2], idx["pe"])
    assert np.array_equal(x[:, 3], idx["ri_slot"])
    assert np.array_equal(x[:, 4], idx["rt"])
    assert np.all(x[:, 5:] == 0)
    # and with the real tables the result is the plain fp64 sum of the five rows
    xr = oracle.embed_sum(oracle_tables(tables), b.hist_items, b.cand_items, idx)
    r = 3
    want = (tables.item.f32()[items[r]].astype(np.float64) + tables.action.f32()[idx["act"][r]]
            + tables.pos.f32()[idx["pe"][r]] + tables.ri.f32()[idx["ri_slot"][r]]
            + tables.rt.f32()[idx["rt"][r]])
    assert np.allclose(xr[r], want, rtol=0, atol=1e-12)
