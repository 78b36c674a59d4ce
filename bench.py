#!/usr/bin/env python3
"""GenRank ranking forward on one MI355X: throughput, per-kernel roofline, CPU-oracle baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload infer_1layer_bf16]

A step is one pass of the hot path over one batch already resident in HBM:
    embed-sum (fused index derivation + five-table gather)
    -> QKV projection -> masked ALiBi attention -> output projection      (single-layer form)
or, for pre-norm workloads, embed-sum -> L x genrank_layer_fwd -> action head.
With --kv-cache a step scores the candidates against cached history keys and values.
With --workload train2_bf16 a step is one training step (forward, BCE at the candidates,
backward, table gradients) and the roofline is the attention backward's.
With --workload hstu_interleaved it instead measures the HSTU-style comparison on the same
users: the interleaved item/action sequence (2N + m slots) with a learned relative bias
materialised in memory, against the action-oriented attention with in-register ALiBi.
Forward workloads: each kernel is timed in a pass of its own with one HIP event pair around
it (on the stream it runs on; events between every launch would add gaps), which also picks
the dominant kernel.  The timed pass then runs exactly --steps steps between device
synchronisations with one event pair around the dominant kernel alone; its wall clock gives
the step time and its events the roofline.  Prints ONE JSON line on stdout; progress goes to
stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "candidates scored/sec (GenRank fwd, bf16) + attn MFMA util % and gather GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
N_XCD, N_SIMD = 8, 256 * 4     # MI355X: 8 XCDs, 256 CUs of 4 SIMDs
KERNEL_SOURCES = {"embed_sum": "embed.hip", "attn_fwd": "attn_fwd.hip", "qkv_gemm": "gemm.hip",
                  "out_gemm": "gemm.hip", "embed": "embed.hip", "norm": "rowops.hip", "qkv": "gemm.hip",
                  "attn": "attn_fwd.hip", "attn_cand": "attn_fwd.hip", "wo": "gemm.hip", "ffn_up": "gemm.hip",
                  "ffn_down": "gemm.hip", "kv": "gemm.hip", "head": "rowops.hip", "attn_bwd": "attn_bwd.hip"}


# --attn-variant -> genrank_alibi.flags (1 = fully visible history, 2 = bucketed time term)
VARIANT_FLAGS = {"causal": 0, "full": 1, "bucket": 2, "both": 3}


def variant_args(args, cfg):
    """(flags, bucket edges or None) of the requested ALiBi variant; the edges are the
    request-gap bucket edges of the workload's time table."""
    import synth
    flags = VARIANT_FLAGS[args.attn_variant]
    return flags, (synth.rt_boundaries(cfg.n_rt) if flags & 2 else None)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="stack4_bf16",
                   help="stack4_bf16 (the 4-layer pre-norm stack, default), infer_1layer_bf16, train2_bf16, "
                        "hstu_interleaved")
    p.add_argument("--no-prune", action="store_true",
                   help="pre-norm stacks: form every row of the top block (by default the top block forms "
                        "the history rows' keys and values only, which is all the logits read)")
    p.add_argument("--chunks", type=int, default=0,
                   help="pre-norm stacks: run the step as this many (>= 1) sequential sub-batches of "
                        "consecutive users (each a whole forward), so that a chunk's intermediate "
                        "tensors can stay in the last-level cache between kernels; whole-step timing "
                        "only")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU-oracle baseline budget (0 disables the leg)")
    p.add_argument("--kv-cache", action="store_true",
                   help="serving: score the candidates against the users' cached history keys/values")
    p.add_argument("--attn-variant", default="causal", choices=sorted(VARIANT_FLAGS),
                   help="ALiBi variant: causal history (default), fully visible history, bucketed "
                        "time bias, or both")
    p.add_argument("--item-dist", choices=["zipf", "uniform"], default=None,
                   help="item id distribution (default: the workload's); uniform ids are the gather's "
                        "control run, where nearly every item row is read once")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="also run one plain device copy of this many MiB (counter calibration)")
    p.add_argument("--units-once", metavar="ORDER_JSON", default=None,
                   help="for counter runs: after the warm-up steps run every unit of "
                        "the step once, in order, write the units' names and kinds to ORDER_JSON, make the "
                        "calibration copy (--calibrate-copy-mb) and stop")
    p.add_argument("--write-traffic", nargs="+", metavar="ARG", default=None,
                   help="host only: ORDER_JSON FETCH_DIR WRITE_DIR [MFMA_DIR]: read the rocprofv3 "
                        "FETCH_SIZE and WRITE_SIZE counter runs of a --units-once run (and optionally its "
                        "SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE run) and store each unit kind's "
                        "per-launch HBM bytes (and MFMA busy share) in profiles/traffic.json")
    return p.parse_args()


def source_sha(fn):
    path = os.path.join(ROOT, "generative_ranking_recommendation_amd", "csrc", fn)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload, field=None):
    """Counter-measured HBM bytes per launch, from committed rocprofv3 summaries; a kernel
    whose source changed since the counters were taken gets None.  field: another value of
    the same records instead (e.g. the MFMA busy share)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    out = {}
    for name, rec in data.get(workload, {}).items():
        src = KERNEL_SOURCES.get(name)
        if src and rec.get("source_sha") == source_sha(src):
            if field is None:
                out[name] = rec["fetch_bytes"] + rec["write_bytes"]
            elif field in rec:
                out[name] = rec[field]
    return out


def cpu_baseline(cfg, batch, tables, weights, budget_s, variant=(0, None)):
    """The fp64 CPU oracle on the first users of the same batch, for about budget_s seconds
    (``variant``: the ALiBi variant's flags and bucket edges)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from common import oracle_geom, oracle_head, oracle_indices, oracle_layers, oracle_tables
    layers = oracle_layers(weights)
    head = oracle_head(weights) if cfg.block == "prenorm" else None
    tabs = oracle_tables(tables)
    t0 = time.perf_counter()
    users = 0
    while users < batch.B and (users < 2 or time.perf_counter() - t0 < budget_s):
        sub = batch.subset([users])
        c1 = cfg.replace(B=1)
        idx = oracle_indices(c1, sub, tables)
        x = oracle.embed_sum(tabs, sub.hist_items, sub.cand_items, idx)
        geom = oracle_geom(c1, sub, idx)
        geom.update(history="full" if variant[0] & 1 else "causal", time_bounds=variant[1])
        oracle.model_fwd(x, layers, cfg.block, cfg.H, geom, head)
        users += 1
    dt = time.perf_counter() - t0
    return {"value": users * cfg.m / dt, "unit": "candidates/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {users} users of {cfg.name} (same seeded batch), full forward "
                      f"in fp64 numpy: indices, embed-sum, {cfg.layers} block(s)"
                      + (", head" if head else "") + f"; {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def bench_hstu(args):
    """Attention cost of the interleaved sequence with a materialised learned bias (HSTU
    style) vs the action-oriented sequence with in-register ALiBi, on the same users (the
    256-user inference batch).  q, k, v are N(0, 1) bf16 of the right shapes: only the
    attention (and the bias materialisation) is compared."""
    import numpy as np
    import torch

    import synth
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    from generative_ranking_recommendation_amd.device import DeviceInputs, to_device
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    base = synth.make_config("infer_1layer_bf16")  # the same data as the inference batch
    cfg = synth.make_config("hstu_interleaved")
    batch = synth.make_batch(base)
    dev = "cuda"
    torch.cuda.set_device(0)
    inp = DeviceInputs(batch, dev)
    d, H, m = cfg.d, cfg.H, base.m
    bt = B.make_batch(inp.B, m, d, H, inp.max_hist, inp.total_hist, B.BF16)
    rng = np.random.default_rng(1000 * cfg.index + 3)
    n_pos, n_time = 1024, 64
    pt = to_device((rng.standard_normal(n_pos) * 0.02).astype(np.float32), dev)
    tt = to_device((rng.standard_normal(n_time) * 0.02).astype(np.float32), dev)
    bounds = to_device(synth.rt_boundaries(n_time), dev, np.int64)
    rab_off = torch.empty(inp.B + 1, dtype=torch.int64, device=dev)
    B.genrank_hstu_rab_layout(bt, inp.hist_offsets, rab_off)
    torch.cuda.synchronize()
    rab_elems = int(rab_off[-1].item())
    rab = torch.empty(rab_elems, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    T1 = inp.total_hist + inp.B * m
    T2 = 2 * inp.total_hist + inp.B * m
    qkv1 = torch.randn((T1, 3 * d), generator=g, device=dev).to(torch.bfloat16)
    qkv2 = torch.randn((T2, 3 * d), generator=g, device=dev).to(torch.bfloat16)
    o1 = torch.empty((T1, d), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty((T2, d), dtype=torch.bfloat16, device=dev)
    l1 = torch.empty((T1, H), dtype=torch.float32, device=dev)
    l2 = torch.empty((T2, H), dtype=torch.float32, device=dev)
    sp, st = alibi_slopes(H, base.time_ratio)
    slopes = B.HostSlopes(sp, st)
    stream = torch.cuda.current_stream()
    es = 2
    p1, p2 = qkv1.data_ptr(), qkv2.data_ptr()
    ops = {
        "hstu_rab": lambda: B.genrank_hstu_rab(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, pt, n_pos, tt,
                                               bounds, n_time, rab_off, rab, stream),
        "hstu_attn": lambda: B.genrank_hstu_attn_fwd(bt, inp.hist_offsets, rab, rab_off, p2, p2 + d * es,
                                                     p2 + 2 * d * es, 3 * d, o2, d, l2, stream),
        "alibi_attn": lambda: B.genrank_attn_fwd(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, slopes, p1,
                                                 p1 + d * es, p1 + 2 * d * es, 3 * d, o1, d, l1, stream),
    }
    times = {}
    for name, fn in ops.items():
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for k in range(args.steps):
            fn()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        times[name] = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)])) * 1e3
        log(f"{name}: {times[name]:.1f} us")
    lengths = inp.lengths
    pairs1 = W.attention_pairs(lengths, m)
    pairs2 = W.attention_pairs(2 * lengths, m)
    rab_bytes = rab_elems * 2
    # learned-bias attention: per (user, head) the bias rows of allowed pairs, read once
    bias_read = H * pairs2 * 2
    out = {
        "metric": "attention time per batch: interleaved sequence + materialised learned bias "
                  "vs action-oriented sequence + in-register ALiBi",
        "value": round(times["hstu_attn"] + times["hstu_rab"], 2),
        "unit": "us",
        "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
        "data": "synthetic: the inference batch's users; q, k, v ~ N(0, 1)",
        "config": {"workload": cfg.name, "users": inp.B, "candidates_per_user": m, "d": d, "heads": H,
                   "bias_tables": {"position_diff": n_pos, "time_diff": n_time}},
        "times_us": {k: round(v, 2) for k, v in times.items()},
        "ratio_hstu_over_alibi": round((times["hstu_attn"] + times["hstu_rab"]) / times["alibi_attn"], 2),
        "ratio_attention_only": round(times["hstu_attn"] / times["alibi_attn"], 2),
        "allowed_pairs": {"interleaved": int(pairs2), "action_oriented": int(pairs1),
                          "ratio": round(pairs2 / pairs1, 3)},
        "flops": {"interleaved": int(W.attention_fwd_flops(2 * lengths, m, d)),
                  "action_oriented": int(W.attention_fwd_flops(lengths, m, d))},
        "bytes": {"bias_written": rab_bytes, "bias_read_allowed_pairs": int(bias_read),
                  "qkv_o_interleaved": int((T2 * 4 * d) * es),
                  "qkv_o_action_oriented": int((T1 * 4 * d) * es)},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_train(cfg, batch, tables, weights, labels, budget_s, variant=(0, None)):
    """The fp64 CPU oracle's training step (forward, BCE at candidates, backward, table
    gradients) on the first users of the same batch, for about budget_s seconds."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from common import oracle_geom, oracle_head, oracle_indices, oracle_layers, oracle_tables
    layers, head, tabs = oracle_layers(weights), oracle_head(weights), oracle_tables(tables)
    t0 = time.perf_counter()
    users = 0
    while users < batch.B and (users < 1 or time.perf_counter() - t0 < budget_s):
        sub = batch.subset([users])
        c1 = cfg.replace(B=1)
        idx = oracle_indices(c1, sub, tables)
        x = oracle.embed_sum(tabs, sub.hist_items, sub.cand_items, idx)
        geom = oracle_geom(c1, sub, idx)
        geom.update(history="full" if variant[0] & 1 else "causal", time_bounds=variant[1])
        xf, logits, caches = oracle.model_fwd(x, layers, cfg.block, cfg.H, geom, head)
        lab = labels[users * cfg.m:(users + 1) * cfg.m]
        oracle.bce_loss(logits, lab)
        dx0, _, _ = oracle.model_bwd(oracle.bce_loss_bwd(logits, lab), xf, layers, cfg.block, cfg.H, geom,
                                     caches, head)
        shapes = {k: getattr(tables, k).shape for k in ("action", "pos", "ri", "rt")}
        used = np.concatenate([sub.hist_items, sub.cand_items])
        shapes["item"] = (int(used.max()) + 1, cfg.d)
        oracle.embed_bwd(dx0, shapes, sub.hist_items, sub.cand_items, idx)
        users += 1
    dt = time.perf_counter() - t0
    return {"value": users * cfg.m / dt, "unit": "candidates/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {users} users of {cfg.name} (same seeded batch), full training step in fp64 "
                      f"numpy: forward, BCE at candidates, backward, table gradients; {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def bench_train(args, cfg):
    """One training step (forward with saved activations, BCE at candidate positions, full
    backward with table gradients) per step; candidates trained per second.  The roofline is
    reported for the attention backward, timed alone on the same batch geometry with
    q, k, v, dO ~ N(0, 1) (two MFMA kernels: dQ, which also forms D, then dK/dV)."""
    import numpy as np
    import torch

    import synth
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    from generative_ranking_recommendation_amd.device import DeviceInputs, to_device
    from generative_ranking_recommendation_amd.model import GenRank
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    log(f"workload {cfg.name}: generating inputs")
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    labels = synth.make_labels(cfg)
    sp, st = alibi_slopes(cfg.H, cfg.time_ratio)
    dev = "cuda"
    torch.cuda.set_device(0)
    vflags, vedges = variant_args(args, cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, dev, attn_flags=vflags, time_bounds=vedges)
    inp = DeviceInputs(batch, dev)
    lab = to_device(labels, dev, np.float32)
    T, d, H, m = inp.rows, cfg.d, cfg.H, cfg.m
    for _ in range(args.warmup):
        model.train_step(inp, lab)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        model.train_step(inp, lab)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"{ms:.4f} ms/step")

    # attention backward alone
    bt = model.batch(inp)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    qkv = torch.randn((T, 3 * d), generator=g, device=dev).to(torch.bfloat16)
    dout = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    dqkv = torch.empty((T, 3 * d), dtype=torch.bfloat16, device=dev)
    nws = B.genrank_workspace_size(B.OP_ATTN_BWD, bt)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    sl = model.layers[0].slopes
    stream = torch.cuda.current_stream()
    p, q = qkv.data_ptr(), dqkv.data_ptr()
    B.genrank_attn_fwd(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, sl, p, p + 2 * d, p + 4 * d, 3 * d,
                       o, d, lse, stream)

    def bwd():
        B.genrank_attn_bwd(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, sl, p, p + 2 * d, p + 4 * d, 3 * d,
                           o, dout, d, lse, q, q + 2 * d, q + 4 * d, 3 * d, 0, ws, nws, stream)
    for _ in range(args.warmup):
        bwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(args.steps):
        bwd()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    t_us = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)])) * 1e3
    if args.units_once:
        # the attention backward once, alone on the device (its dQ and dK/dV dispatches), then
        # the calibration copy
        if args.calibrate_copy_mb > 0:
            src = torch.ones(args.calibrate_copy_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
        torch.cuda.synchronize()
        bwd()
        torch.cuda.synchronize()
        with open(args.units_once, "w") as f:
            json.dump({"workload": cfg.name, "units": [["attn_bwd", "attn_bwd", 2]],
                       "copy_mib": args.calibrate_copy_mb}, f)
        if args.calibrate_copy_mb > 0:
            dst.copy_(src)
            torch.cuda.synchronize()
        log(f"units once: the attention backward; order in {args.units_once}")
        return
    lengths = inp.lengths
    flops = W.attention_bwd_flops(lengths, m, d, full_history=bool(vflags & 1))
    flops_rc = W.attention_bwd_flops(lengths, m, d, recompute=True, full_history=bool(vflags & 1))
    nbytes = W.attention_bwd_hbm_floor_bytes(T, d, H)
    if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12):
        bound, achieved, peak, unit = "hbm", nbytes / (t_us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / (t_us * 1e-6) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    tf = flops / (t_us * 1e-6) / 1e12
    log(f"attention backward {t_us:.1f} us, {tf:.1f} TFLOP/s (recompute excluded)")
    traffic = load_traffic(cfg.name).get("attn_bwd") if args.attn_variant == "causal" else None
    roofline = {"kernel": "attn_bwd", "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic}
    cpu = None
    if args.cpu_seconds > 0:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline_train(cfg, batch, tables, weights, labels, args.cpu_seconds, (vflags, vedges))
        log(f"CPU oracle: {cpu['value']:.1f} candidates/s on {cpu['cores']} threads")
    out = {
        "metric": "candidates trained/sec (GenRank fwd + bwd, bf16)",
        "value": round(inp.B * m / (ms * 1e-3), 1),
        "unit": "candidates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; Zipf(1.1) item ids, jagged histories, Bernoulli(0.1) labels)",
        "config": {"workload": cfg.name, "users": inp.B, "candidates_per_user": m,
                   "history": f"U[{cfg.hist_min},{cfg.hist_max}]", "rows": T, "d": d, "heads": H,
                   "layers": cfg.layers, "block": cfg.block, "attn_variant": args.attn_variant},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": {"attn_bwd": {"time_us": round(t_us, 2), "bound": bound, "achieved": round(achieved, 2),
                                 "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                                 "flops": int(flops), "flops_with_recompute": int(flops_rc),
                                 "floor_bytes": int(nbytes), "tflops": round(tf, 2),
                                 "mfma_util_pct": round(100 * tf / PEAK_BF16_TFLOPS, 2)}},
    }
    print(json.dumps(out), flush=True)


def bench_serve(args, cfg):
    """Serving with cached history: the users' history keys and values are computed once
    (prefill, timed and reported on its own); a step scores the request's candidates only:
    embed the candidate rows -> QKV of those rows -> candidate attention against the cached
    history K/V (plus each candidate's own key) -> output projection."""
    import numpy as np
    import torch

    import synth
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    from generative_ranking_recommendation_amd.device import DeviceInputs
    from generative_ranking_recommendation_amd.model import GenRank
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    if not (cfg.block == "attn_only" and cfg.layers == 1 and cfg.dtype == "bf16"):
        print("--kv-cache measures the single-layer bf16 form", file=sys.stderr)
        sys.exit(2)
    log(f"workload {cfg.name} (cached history): generating inputs")
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    sp, st = alibi_slopes(cfg.H, cfg.time_ratio)
    dev = "cuda"
    torch.cuda.set_device(0)
    vflags, vedges = variant_args(args, cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, dev, attn_flags=vflags, time_bounds=vedges)
    inp = DeviceInputs(batch, dev)
    T_h, d, H, m = inp.total_hist, cfg.d, cfg.H, cfg.m
    Tc = inp.B * m
    bt = model.batch(inp)
    lay = model.layers[0]
    stream = torch.cuda.current_stream()
    # prefill: the history keys and values
    for _ in range(2):
        caches = model.prefill(inp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        caches = model.prefill(inp)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t0) * 1e3 / 5
    kv = caches[0]
    xc = torch.empty((Tc, d), dtype=torch.bfloat16, device=dev)
    qkv = torch.empty((Tc, 3 * d), dtype=torch.bfloat16, device=dev)
    o = torch.empty((Tc, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((Tc, d), dtype=torch.bfloat16, device=dev)
    qp, kp = qkv.data_ptr(), kv.data_ptr()
    names = ["embed_cand", "qkv_gemm", "attn_cached", "out_gemm"]
    launches_on = lambda st: [
        lambda: B.genrank_embed_sum_cand(bt, inp.struct, model.tables.struct, xc, st),
        lambda: B.genrank_linear(B.BF16, xc, d, lay.wqkv, d, qkv, 3 * d, Tc, 3 * d, d, stream=st),
        lambda: B.genrank_attn_fwd_cached(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, lay.slopes, qp,
                                          qp + 2 * d, qp + 4 * d, 3 * d, kp, kp + 2 * d, 2 * d, o, d, None,
                                          st),
        lambda: B.genrank_linear(B.BF16, o, d, lay.wo, d, y, d, Tc, d, d, stream=st),
    ]
    launches = launches_on(stream)

    def step(ev=None, only=None):
        """Events after every launch (breakdown), or one pair around launch ``only``."""
        if ev is not None and only is None:
            ev[0].record(stream)
        for i, fn in enumerate(launches):
            if i == only:
                ev[0].record(stream)
            fn()
            if ev is not None and only is None:
                ev[i + 1].record(stream)
            if i == only:
                ev[1].record(stream)
    mk = lambda k: [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the scored rows must equal the candidate rows of the full forward
    y_full, _ = model.forward(inp)
    torch.cuda.synchronize()
    if not torch.equal(y_full[T_h:], y):
        log("WARNING: cached scoring differs from the full forward")
    # per-kernel passes (one event pair around one launch), then the timed pass with one
    # event pair around the cached attention
    per = {}
    for i, n in enumerate(names):
        events = [mk(2) for _ in range(args.steps)]
        for k in range(args.steps):
            step(events[k], only=i)
        torch.cuda.synchronize()
        per[n] = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    events = [mk(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], only=2)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    per["attn_cached"] = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    log(f"{ms_eager:.4f} ms/step launched one call at a time; kernels (ms): " +
        ", ".join(f"{k}={v:.4f}" for k, v in per.items()))
    # the timed step: the four launches captured once in a HIP graph and replayed, so that
    # the host enqueues one graph per request batch instead of four calls (the same kernels,
    # arguments and buffers; a replay must reproduce the eager rows bit for bit)
    y_eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for fn in launches_on(cap):
            fn()
    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(y, y_eager))
    if not graph_same:
        log("WARNING: the graph replay differs from the eager step")
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"{ms:.4f} ms/step replayed as one graph (equal to the eager rows: {graph_same})")
    lengths = inp.lengths
    cand_pairs = int(m * (np.asarray(lengths, np.int64) + 1).sum())
    flops = 4 * d * cand_pairs
    nbytes = T_h * 2 * d * 2 + Tc * 3 * d * 2 + Tc * d * 2
    t_us = per["attn_cached"] * 1e3
    achieved = nbytes / (t_us * 1e-6) / 1e9
    roofline = {"kernel": "attn_cached", "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    kernels = {n: {"time_us": round(v * 1e3, 2)} for n, v in per.items()}
    kernels["attn_cached"].update({"bound": "hbm", "achieved": round(achieved, 2), "floor_bytes": int(nbytes),
                                   "flops": int(flops),
                                   "tflops": round(flops / (t_us * 1e-6) / 1e12, 2)})
    cpu = None
    if args.cpu_seconds > 0:
        log("CPU oracle baseline (the oracle's full forward: it keeps no cache) ...")
        cpu = cpu_baseline(cfg, batch, tables, weights, args.cpu_seconds, (vflags, vedges))
        log(f"CPU oracle: {cpu['value']:.1f} candidates/s on {cpu['cores']} threads")
    out = {
        "metric": "candidates scored/sec with cached history K/V (GenRank fwd, bf16)",
        "value": round(Tc / (ms * 1e-3), 1),
        "unit": "candidates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; Zipf(1.1) item ids, jagged histories, runs of 1-4 actions per request)",
        "config": {"workload": cfg.name, "mode": "cached history", "users": inp.B, "candidates_per_user": m,
                   "history": f"U[{cfg.hist_min},{cfg.hist_max}]", "history_rows": T_h, "d": d, "heads": H,
                   "attn_variant": args.attn_variant},
        "prefill_ms": round(prefill_ms, 4),
        "ms_per_step_eager": round(ms_eager, 5),
        "step_launch": "HIP graph replay of the step's four launches",
        "graph_equals_eager": graph_same,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def stack_units(model, inp, bufs, prune=True):
    """The pre-norm stack's forward as a chain of C-ABI calls, one per kernel-sized unit:
    embed -> per block [norm, QKV, attention, output projection + residual, norm, FFN up +
    SiLU, FFN down + residual] -> head at the candidate rows.  With ``prune`` the top block
    forms only what the logits read: the history rows' keys and values, then the candidate
    rows' block (their queries attend the history K/V and themselves); its history outputs
    are never formed.  Returns [(name, kind, fn, (bound, amount, unit))]."""
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    x, z, qkv, o, x1, hdn, kv, logits = (bufs[k] for k in ("x", "z", "qkv", "o", "x1", "hdn", "kv", "logits"))
    bt = model.batch(inp)
    bc = B.make_batch(inp.B, inp.m, model.d, model.H, 0, 0, model.code, model.resid)  # candidate rows only
    T, T_h, d, H, m = inp.rows, inp.total_hist, model.d, model.H, inp.m
    Tc = inp.B * m
    rc, ac = model.resid_code, model.code
    es, rs = (2 if ac == B.BF16 else 4), (4 if rc == B.F32 else 2)
    stream = torch_stream()
    ptr = lambda t, rows=0, cols=0, ld=None: t.data_ptr() + (rows * (ld or t.shape[-1]) + cols) * t.element_size()
    gemm = lambda M, N, K, out_es=es, res_es=0: ("mfma", W.gemm_flops(M, N, K), "TFLOP/s")
    norm = lambda rows: ("hbm", rows * d * (rs + es) + d * 4, "GB/s")
    units = []
    uniq = int(np.unique(np.concatenate([inp.host.hist_items, inp.host.cand_items])).size)
    tabs = model.tables
    small_rows = int(tabs.action.shape[0] + tabs.pos.shape[0] + tabs.ri.shape[0] + tabs.rt.shape[0])
    idx_bytes = T_h * (4 + 4 + 8) + Tc * 4 + (inp.B + 1) * 4 + inp.B * 8
    gbytes = T * d * rs + uniq * d * es + small_rows * d * es + idx_bytes
    units.append(("embed", "embed", lambda: B.genrank_embed_sum(bt, inp.struct, tabs.struct, x, stream),
                  ("hbm", gbytes, "GB/s")))
    L = len(model.layers)
    lengths = inp.lengths
    attn_flops = W.attention_fwd_flops(lengths, m, d)
    # a forward that serves no backward stores no softmax statistics
    attn_bytes = T * 3 * d * es + T * d * es
    cand_attn_flops = 4 * d * int(m * (np.asarray(lengths, np.int64) + 1).sum())
    cand_attn_bytes = T_h * 2 * d * es + Tc * 3 * d * es + Tc * d * es

    def attn_work(flops, nbytes):
        if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12):
            return ("hbm", nbytes, "GB/s")
        return ("mfma", flops, "TFLOP/s")

    for i, lay in enumerate(model.layers):
        F = lay.ffn_dim
        sl = lay.slopes
        top = prune and i == L - 1
        pre = f"L{i}."
        if not top:
            q = qkv.data_ptr()
            units += [
                (pre + "norm1", "norm", lambda lay=lay: B.genrank_rmsnorm(rc, ac, x, lay.g1, z, T, d, stream), norm(T)),
                (pre + "qkv", "qkv", lambda lay=lay: B.genrank_linear(ac, z, d, lay.wqkv, d, qkv, 3 * d, T, 3 * d, d,
                                                                      stream=stream), gemm(T, 3 * d, d)),
                (pre + "attn", "attn", lambda sl=sl, q=q: B.genrank_attn_fwd(bt, inp.hist_offsets, inp.hist_ts,
                                                                              inp.req_ts, sl, q, q + d * es,
                                                                              q + 2 * d * es, 3 * d, o, d, None,
                                                                              stream), attn_work(attn_flops, attn_bytes)),
                (pre + "wo", "wo", lambda lay=lay: B.genrank_linear(ac, o, d, lay.wo, d, x1, d, T, d, d,
                                                                    epilogue=B.EPI_RESIDUAL_F32 if rc == B.F32
                                                                    else B.EPI_RESIDUAL, residual=x, ldr=d,
                                                                    stream=stream), gemm(T, d, d)),
                (pre + "norm2", "norm", lambda lay=lay: B.genrank_rmsnorm(rc, ac, x1, lay.g2, z, T, d, stream), norm(T)),
                (pre + "ffn_up", "ffn_up", lambda lay=lay, F=F: B.genrank_linear(ac, z, d, lay.w1, d, hdn, F, T, F, d,
                                                                                 epilogue=B.EPI_SILU, stream=stream),
                 gemm(T, F, d)),
                (pre + "ffn_down", "ffn_down", lambda lay=lay, F=F: B.genrank_linear(
                    ac, hdn, F, lay.w2, F, x, d, T, d, F, epilogue=B.EPI_RESIDUAL_F32 if rc == B.F32 else B.EPI_RESIDUAL,
                    residual=x1, ldr=d, stream=stream), gemm(T, d, F)),
            ]
            continue
        # top block: history keys and values, then the candidate rows alone
        xc, zc, oc, x1c, hc = ptr(x, T_h), z.data_ptr(), o.data_ptr(), x1.data_ptr(), hdn.data_ptr()
        q = qkv.data_ptr()
        wkv = lay.wqkv.data_ptr() + d * d * es
        kvp = kv.data_ptr()
        units += [
            (pre + "norm1_hist", "norm", lambda lay=lay: B.genrank_rmsnorm(rc, ac, x, lay.g1, z, T_h, d, stream),
             norm(T_h)),
            (pre + "kv_hist", "kv", lambda: B.genrank_linear(ac, z, d, wkv, d, kv, 2 * d, T_h, 2 * d, d, stream=stream),
             gemm(T_h, 2 * d, d)),
            (pre + "norm1", "norm", lambda lay=lay, xc=xc: B.genrank_rmsnorm(rc, ac, xc, lay.g1, zc, Tc, d, stream),
             norm(Tc)),
            (pre + "qkv", "qkv", lambda lay=lay: B.genrank_linear(ac, zc, d, lay.wqkv, d, q, 3 * d, Tc, 3 * d, d,
                                                                  stream=stream), gemm(Tc, 3 * d, d)),
            (pre + "attn", "attn_cand", lambda sl=sl: B.genrank_attn_fwd_cached(
                bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, sl, q, q + d * es, q + 2 * d * es, 3 * d, kvp,
                kvp + d * es, 2 * d, oc, d, None, stream), attn_work(cand_attn_flops, cand_attn_bytes)),
            (pre + "wo", "wo", lambda lay=lay, xc=xc: B.genrank_linear(
                ac, oc, d, lay.wo, d, x1c, d, Tc, d, d, epilogue=B.EPI_RESIDUAL_F32 if rc == B.F32 else B.EPI_RESIDUAL,
                residual=xc, ldr=d, stream=stream), gemm(Tc, d, d)),
            (pre + "norm2", "norm", lambda lay=lay: B.genrank_rmsnorm(rc, ac, x1c, lay.g2, zc, Tc, d, stream), norm(Tc)),
            (pre + "ffn_up", "ffn_up", lambda lay=lay, F=F: B.genrank_linear(ac, zc, d, lay.w1, d, hc, F, Tc, F, d,
                                                                             epilogue=B.EPI_SILU, stream=stream),
             gemm(Tc, F, d)),
            (pre + "ffn_down", "ffn_down", lambda lay=lay, F=F, xc=xc: B.genrank_linear(
                ac, hc, F, lay.w2, F, xc, d, Tc, d, F, epilogue=B.EPI_RESIDUAL_F32 if rc == B.F32 else B.EPI_RESIDUAL,
                residual=x1c, ldr=d, stream=stream), gemm(Tc, d, F)),
        ]
    head = model.head
    xh = ptr(x, T_h) if prune else x
    hb = bc if prune else bt
    units.append(("head", "head", lambda: B.genrank_head_fwd(hb, xh, head.g_final, head.w_head, head.b_head,
                                                             head.n_tasks, logits, stream),
                  ("hbm", Tc * d * rs + Tc * head.n_tasks * 4, "GB/s")))
    return units


def torch_stream():
    import torch
    return torch.cuda.current_stream()


def bench_stack_chunked(args, cfg):
    """The stack step as --chunks sequential forwards over sub-batches of consecutive users
    (users are independent, so the logits equal the whole batch's), each the decomposed
    pruned forward of bench_stack; candidates scored per second over the whole batch."""
    import torch

    import synth
    from generative_ranking_recommendation_amd.device import DeviceInputs
    from generative_ranking_recommendation_amd.model import GenRank
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    log(f"workload {cfg.name}: generating inputs ({args.chunks} chunks)")
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    sp, st = alibi_slopes(cfg.H, cfg.time_ratio)
    dev = "cuda"
    torch.cuda.set_device(0)
    vflags, vedges = variant_args(args, cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, dev, attn_flags=vflags, time_bounds=vedges)
    bounds = np.linspace(0, batch.B, args.chunks + 1).round().astype(int)
    units, logits = [], []
    for c in range(args.chunks):
        sub = batch.subset(range(bounds[c], bounds[c + 1]))
        inp = DeviceInputs(sub, dev)
        bufs = stack_bufs(model, inp, dev)
        logits.append(bufs["logits"])
        units += [(f"c{c}.{n}", kind, fn, w) for n, kind, fn, w in stack_units(model, inp, bufs)]
    Tc = batch.B * cfg.m
    log(f"{len(units)} launches per step")

    def step():
        for _, _, fn, _ in units:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    got = torch.cat(logits)
    _, ref = model.forward(DeviceInputs(batch, dev))
    torch.cuda.synchronize()
    same = bool(torch.equal(got, ref))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"{ms:.4f} ms/step in {args.chunks} chunks; logits equal to the whole batch's: {same}")
    out = {"metric": METRIC, "value": round(Tc / (ms * 1e-3), 1), "unit": "candidates/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
           "config": {"workload": cfg.name, "users": batch.B, "chunks": args.chunks,
                      "users_per_chunk": [int(b - a) for a, b in zip(bounds[:-1], bounds[1:])]},
           "logits_equal_forward": same, "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def stack_bufs(model, inp, dev):
    """Device buffers of the decomposed stack forward for one batch."""
    import torch
    T, T_h, d = inp.rows, inp.total_hist, model.d
    F = model.layers[0].ffn_dim
    bf = torch.bfloat16
    return {"x": model.resid_rows(T), "z": torch.empty((T, d), dtype=bf, device=dev),
            "qkv": torch.empty((T, 3 * d), dtype=bf, device=dev), "o": torch.empty((T, d), dtype=bf, device=dev),
            "x1": model.resid_rows(T), "hdn": torch.empty((T, F), dtype=bf, device=dev),
            "kv": torch.empty((T_h, 2 * d), dtype=bf, device=dev),
            "logits": torch.empty((inp.B * inp.m, model.head.n_tasks), dtype=torch.float32, device=dev)}


def bench_stack(args, cfg):
    """The full pre-norm stack forward (embed -> L blocks -> action head), each kernel-sized
    unit a C-ABI call of its own on one stream; candidates scored per second."""
    import torch
    if args.chunks >= 1:
        return bench_stack_chunked(args, cfg)

    import synth
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    from generative_ranking_recommendation_amd.device import DeviceInputs
    from generative_ranking_recommendation_amd.model import GenRank
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    log(f"workload {cfg.name}: generating inputs")
    batch, tables, weights = synth.make_batch(cfg), synth.make_tables(cfg), synth.make_weights(cfg)
    sp, st = alibi_slopes(cfg.H, cfg.time_ratio)
    dev = "cuda"
    torch.cuda.set_device(0)
    vflags, vedges = variant_args(args, cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, dev, attn_flags=vflags, time_bounds=vedges)
    inp = DeviceInputs(batch, dev)
    T, T_h, d, H, m = inp.rows, inp.total_hist, cfg.d, cfg.H, cfg.m
    Tc = inp.B * m
    F = model.layers[0].ffn_dim
    bufs = stack_bufs(model, inp, dev)
    log(f"T={T} rows (history {T_h}, candidates {Tc}); uploading done")
    prune = not args.no_prune
    units = stack_units(model, inp, bufs, prune=prune)
    stream = torch.cuda.current_stream()
    names = [u[0] for u in units]

    def step(ev=None, only=None):
        for n, _, fn, _ in units:
            if n == only:
                ev[0].record(stream)
            fn()
            if n == only:
                ev[1].record(stream)

    mk = lambda k: [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.units_once:
        # one launch per unit, in step order, each alone on the device; then the copy (its
        # buffers filled beforehand, so that no other kernel runs between the units and it)
        if args.calibrate_copy_mb > 0:
            src = torch.ones(args.calibrate_copy_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for n, _, fn, _ in units:
            fn()
            torch.cuda.synchronize()
        with open(args.units_once, "w") as f:
            json.dump({"workload": cfg.name, "units": [[n, kind] for n, kind, _, _ in units],
                       "copy_mib": args.calibrate_copy_mb}, f)
        if args.calibrate_copy_mb > 0:
            dst.copy_(src)
            torch.cuda.synchronize()
        log(f"units once: {len(units)} launches; order in {args.units_once}")
        return
    # the decomposed (and pruned) step must give the logits of the model's own forward
    got = bufs["logits"].clone()
    _, ref = model.forward(inp)
    torch.cuda.synchronize()
    same = bool(torch.equal(got, ref))
    if not same:
        log(f"WARNING: the decomposed step's logits differ from the forward's (max "
            f"{(got - ref).abs().max().item():.3g})")
    # the unpruned forward (every block over every row, one genrank_layer_fwd per block)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_ref = max(3, args.steps // 4)
    for _ in range(n_ref):
        model.forward(inp)
    torch.cuda.synchronize()
    ms_unpruned = (time.perf_counter() - t0) * 1e3 / n_ref
    # per-unit passes: --steps steps with one event pair around one unit
    per = {}
    for n in names:
        events = [mk(2) for _ in range(args.steps)]
        for k in range(args.steps):
            step(events[k], only=n)
        torch.cuda.synchronize()
        per[n] = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    traffic = load_traffic(cfg.name) if args.item_dist is None else {}

    def rate(work, t_ms, kind=None):
        bound, amount, unit = work
        if unit == "GB/s":
            achieved, peak = amount / (t_ms * 1e-3) / 1e9, PEAK_HBM_GBS
        else:
            achieved, peak = amount / (t_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS
        return {"time_us": round(t_ms * 1e3, 2), "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "algorithmic": int(amount),
                "traffic": traffic.get(kind)}
    # by kind: total time per step and the launches
    kinds = {}
    for n, kind, _, work in units:
        k = kinds.setdefault(kind, {"launches": [], "time_us": 0.0})
        k["launches"].append(n)
        k["time_us"] += per[n] * 1e3
    dominant_kind = max(kinds, key=lambda k: kinds[k]["time_us"])
    dom = kinds[dominant_kind]["launches"][0]
    dom_work = next(w for n, _, _, w in units if n == dom)
    # timed pass: exactly --steps steps between two device synchronisations, one event pair
    # around the dominant kind's first launch
    events = [mk(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], only=dom)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    t_dom = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    log(f"{ms:.4f} ms/step (unpruned forward {ms_unpruned:.4f} ms); {dom} {t_dom * 1e3:.1f} us in the timed pass")
    kd = rate(dom_work, t_dom, dominant_kind)
    roofline = {"kernel": f"{dominant_kind} ({dom})", "bound": kd["bound"], "achieved": kd["achieved"],
                "peak": kd["peak"], "unit": kd["unit"], "frac": kd["frac"], "traffic": kd["traffic"]}
    units_out = {n: rate(w, per[n], kind) for n, kind, _, w in units}
    kinds_out = {k: {"time_us_per_step": round(v["time_us"], 1), "launches": len(v["launches"]),
                     "share": round(v["time_us"] / (ms * 1e3), 4)} for k, v in kinds.items()}
    floor_us = sum((w[1] / (PEAK_HBM_GBS * 1e9) if w[2] == "GB/s" else w[1] / (PEAK_BF16_TFLOPS * 1e12)) * 1e6
                   for _, _, _, w in units)
    a0 = units_out["L0.attn"]
    attn_flops = W.attention_fwd_flops(inp.lengths, m, d)
    attn_tf = attn_flops / (a0["time_us"] * 1e-6) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(cfg, batch, tables, weights, args.cpu_seconds, (vflags, vedges))
        log(f"CPU oracle: {cpu['value']:.1f} candidates/s on {cpu['cores']} threads")
    out = {
        "metric": METRIC,
        "value": round(Tc / (ms * 1e-3), 1),
        "unit": "candidates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; Zipf(1.1) item ids, jagged histories, runs of 1-4 actions per request)",
        "config": {"workload": cfg.name, "users": inp.B, "candidates_per_user": m,
                   "history": f"U[{cfg.hist_min},{cfg.hist_max}]", "rows": T, "d": d, "heads": H,
                   "layers": cfg.layers, "ffn": F, "block": cfg.block, "attn_variant": args.attn_variant,
                   "residual_stream": "f32" if model.resid == B.RESID_F32 else cfg.dtype,
                   "top_block": "history rows: keys and values only; candidate rows: the whole block"
                   if prune else "every row", "item_dist": cfg.item_dist},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ms_per_step_unpruned": round(ms_unpruned, 4),
        "logits_equal_forward": same,
        "kinds": kinds_out,
        "kernels": units_out,
        "kernel_timing": "each unit: its own pass of --steps steps with one event pair around it; the "
                         "dominant unit: the event pair in the timed pass",
        "attn_mfma_util_pct": round(100 * attn_tf / PEAK_BF16_TFLOPS, 2),
        # the same from rocprofv3 counters of layer 0's attention launch: MFMA busy cycles
        # over (SIMDs x the launch's cycles), None while the source differs from the profile's
        "attn_mfma_busy_pct_counters": load_traffic(cfg.name, "mfma_busy_pct").get("attn"),
        "attn_tflops": round(attn_tf, 2),
        "step_roofline_us": round(floor_us, 1),
        "step_roofline_frac": round(floor_us / (ms * 1e3), 4),
        "gather_gbps": units_out["embed"]["achieved"],
    }
    print(json.dumps(out), flush=True)


def write_traffic(order_json, fetch_dir, write_dir, mfma_dir=None, out_path=None):
    """profiles/traffic.json from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) of
    `bench.py --units-once ... --calibrate-copy-mb N`: the dispatches that precede the
    calibration copy are the step's units in order; each counter is scaled by what it reads
    for the copy (N MiB each way), and each kind keeps the bytes of its first launch."""
    import csv
    import glob

    def short(kernel):  # "void genrank::(anonymous namespace)::k<...>(args)" -> "k<...>"
        return kernel.replace("genrank::(anonymous namespace)::", "").rsplit("(", 1)[0].replace("void ", "")
    with open(order_json) as f:
        order = json.load(f)
    # [name, kind] or [name, kind, dispatches]: a unit of several dispatches sums their counters
    counts = [u[2] if len(u) > 2 else 1 for u in order["units"]]
    units = [u[:2] for u in order["units"]]
    n_disp = sum(counts)

    def group(ds):
        out, i = [], 0
        for c in counts:
            out.append([" + ".join(dict.fromkeys(n for n, _ in ds[i:i + c])), sum(v for _, v in ds[i:i + c])])
            i += c
        return out

    def dispatches(d, counter=None):
        rows = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if counter is None or r["Counter_Name"] == counter:
                        rows.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        return [rows[k] for k in sorted(rows)]
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        ds = dispatches(d)
        ci = max(i for i, (name, _) in enumerate(ds) if "copyBuffer" in name or "copy" in name.lower())
        copy_kib = ds[ci][1]
        out[counter] = (copy_kib, group(ds[ci - n_disp:ci]))
    fetch_copy, fetch_units = out["FETCH_SIZE"]
    write_copy, write_units = out["WRITE_SIZE"]
    mib = order.get("copy_mib")
    moved_kib = float(mib) * 1024 if mib else None
    fs = moved_kib / fetch_copy if moved_kib else 1.0
    wscale = moved_kib / write_copy if moved_kib else 1.0
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    rec = {}
    for (n, kind), (kn, fk), (_, wk) in zip(units, fetch_units, write_units):
        src = KERNEL_SOURCES.get(kind)
        if kind in rec or not src:
            continue
        rec[kind] = {"unit": n, "kernel": " + ".join(short(x) for x in kn.split(" + ")), "source_sha": source_sha(src),
                     "fetch_bytes": int(fk * 1024 * fs), "write_bytes": int(wk * 1024 * wscale),
                     "fetch_kib_raw": int(fk), "write_kib_raw": int(wk)}
    if mfma_dir:
        # MFMA busy share of a launch: SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs (16
        # cycles per 16 x 16 x 32 bf16 MFMA); GRBM_GUI_ACTIVE over the XCDs, each counting the
        # launch's cycles once
        busy, gui = dispatches(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES"), dispatches(mfma_dir, "GRBM_GUI_ACTIVE")
        ci = max(i for i, (name, _) in enumerate(busy) if "copy" in name.lower())
        busy_u, gui_u = group(busy[ci - n_disp:ci]), group(gui[ci - n_disp:ci])
        for (n, kind), (_, b), (_, g) in zip(units, busy_u, gui_u):
            if kind in rec and rec[kind]["unit"] == n and g > 0:
                cycles = g / N_XCD
                rec[kind]["mfma_busy_cycles"] = int(b)
                rec[kind]["gui_active_cycles"] = int(g)
                rec[kind]["mfma_busy_pct"] = round(100.0 * b / (N_SIMD * cycles), 2)
    rec["calibration"] = {"fetch_scale": fs, "write_scale": wscale,
                          "copy": f"torch device copy of {mib} MiB ({fetch_copy:.0f} KiB FETCH_SIZE, "
                                  f"{write_copy:.0f} KiB WRITE_SIZE)"}
    data[order["workload"]] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    for (n, kind), (kn, _) in zip(units, fetch_units):
        print(f"{n:16s} {kind:10s} {' + '.join(short(x) for x in kn.split(' + '))}")
    for kind, r in rec.items():
        if kind != "calibration":
            print(f"{kind:10s} {r['unit']:14s} read {r['fetch_bytes'] / 1e6:9.1f} MB  write {r['write_bytes'] / 1e6:9.1f} MB")


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.workload == "hstu_interleaved":
        bench_hstu(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the GenRank hot path on a single "
              "MI355X (users shard across GPUs with no exchange in the forward; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from generative_ranking_recommendation_amd import binding as B
    from generative_ranking_recommendation_amd import workload as W
    from generative_ranking_recommendation_amd.device import DeviceInputs
    from generative_ranking_recommendation_amd.model import GenRank
    from generative_ranking_recommendation_amd.slopes import alibi_slopes

    cfg = synth.make_config(args.workload)
    if args.item_dist is not None:
        cfg = cfg.replace(item_dist=args.item_dist)
    if cfg.train:
        bench_train(args, cfg)
        return
    if args.kv_cache:
        bench_serve(args, cfg)
        return
    if cfg.block == "prenorm":
        bench_stack(args, cfg)
        return
    log(f"workload {cfg.name}: generating inputs")
    batch = synth.make_batch(cfg)
    tables = synth.make_tables(cfg)
    weights = synth.make_weights(cfg)
    if cfg.slopes_pos is not None:
        sp, st = np.asarray(cfg.slopes_pos, np.float32), np.asarray(cfg.slopes_time, np.float32)
    else:
        sp, st = alibi_slopes(cfg.H, cfg.time_ratio)

    dev = "cuda"
    torch.cuda.set_device(0)
    vflags, vedges = variant_args(args, cfg)
    model = GenRank.from_host(cfg, tables, weights, sp, st, dev, attn_flags=vflags, time_bounds=vedges)
    inp = DeviceInputs(batch, dev)
    T, d, H, m = inp.rows, cfg.d, cfg.H, cfg.m
    bt = model.batch(inp)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4
    code = B.BF16 if cfg.dtype == "bf16" else B.F32
    stream = torch.cuda.current_stream()
    log(f"T={T} rows (history {inp.total_hist}, candidates {inp.B * m}); uploading done")

    x = torch.empty((T, d), dtype=tdt, device=dev)
    decomposed = cfg.block == "attn_only" and cfg.layers == 1
    if decomposed:
        lay = model.layers[0]
        qkv = torch.empty((T, 3 * d), dtype=tdt, device=dev)
        o = torch.empty((T, d), dtype=tdt, device=dev)
        y = torch.empty((T, d), dtype=tdt, device=dev)
        qp = qkv.data_ptr()
        units = [
            ("embed_sum", lambda: B.genrank_embed_sum(bt, inp.struct, model.tables.struct, x, stream)),
            ("qkv_gemm", lambda: B.genrank_linear(code, x, d, lay.wqkv, d, qkv, 3 * d, T, 3 * d, d, stream=stream)),
            ("attn_fwd", lambda: B.genrank_attn_fwd(bt, inp.hist_offsets, inp.hist_ts, inp.req_ts, lay.slopes, qp,
                                                    qp + d * es, qp + 2 * d * es, 3 * d, o, d, None, stream)),
            ("out_gemm", lambda: B.genrank_linear(code, o, d, lay.wo, d, y, d, T, d, d, stream=stream)),
        ]
    else:
        logits = torch.empty((inp.B * m, 4), dtype=torch.float32, device=dev)
        units = [("embed_sum", lambda: B.genrank_embed_sum(bt, inp.struct, model.tables.struct, x, stream))]
        units += [(f"layer{i}", (lambda i=i: model.layer(i, inp, x, x, False, stream))) for i in range(cfg.layers)]
        if model.head:
            units.append(("head", lambda: B.genrank_head_fwd(bt, x, model.head.g_final, model.head.w_head,
                                                             model.head.b_head, model.head.n_tasks, logits, stream)))
    names = [n for n, _ in units]

    def step(ev=None, only=None):
        """One pass of the path.  With ``only`` None and events: an event before the first
        launch and after each (the per-kernel breakdown); with ``only`` a unit's name: one
        event pair around that unit alone (the timed pass)."""
        if ev is not None and only is None:
            ev[0].record(stream)
        for i, (n, fn) in enumerate(units):
            if n == only:
                ev[0].record(stream)
            fn()
            if ev is not None and only is None:
                ev[i + 1].record(stream)
            if n == only:
                ev[1].record(stream)

    mk = lambda k: [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if decomposed:
        # the decomposed step runs the same kernels as genrank_layer_fwd: check it
        y_ref = torch.empty_like(y)
        model.layer(0, inp, x, y_ref, False, stream)
        torch.cuda.synchronize()
        if not torch.equal(y_ref, y):
            log("WARNING: decomposed step differs from genrank_layer_fwd")
    if args.units_once:
        # as for the stacks: every unit once, alone, then the calibration copy
        if args.calibrate_copy_mb > 0:
            src = torch.ones(args.calibrate_copy_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _, fn in units:
            fn()
            torch.cuda.synchronize()
        with open(args.units_once, "w") as f:
            json.dump({"workload": cfg.name, "units": [[n, n] for n in names], "copy_mib": args.calibrate_copy_mb}, f)
        if args.calibrate_copy_mb > 0:
            dst.copy_(src)
            torch.cuda.synchronize()
        log(f"units once: {len(units)} launches; order in {args.units_once}")
        return
    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy_mb} MiB done")

    # per-kernel passes: --steps steps with one event pair around one launch (events
    # between every launch would add gaps and inflate each kernel's figure)
    per = {}
    for n in names:
        events = [mk(2) for _ in range(args.steps)]
        for k in range(args.steps):
            step(events[k], only=n)
        torch.cuda.synchronize()
        per[n] = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    log("per kernel (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in per.items()))

    # algorithmic work per launch
    lengths = inp.lengths
    uniq = int(np.unique(np.concatenate([batch.hist_items, batch.cand_items])).size)
    small_rows = (cfg.n_action + 1) + cfg.n_pos + cfg.n_ri + cfg.n_rt
    idx_bytes = inp.total_hist * (4 + 4 + 8) + inp.B * m * 4 + (inp.B + 1) * 4 + inp.B * 8
    gather_bytes = W.gather_compulsory_bytes(T, d, es, uniq, small_rows, idx_bytes)
    work = {"embed_sum": ("hbm", gather_bytes, "GB/s")}
    attn_flops = None
    if decomposed:
        # attention: algorithmic flops over allowed pairs, and the floor bytes (Q, K, V read
        # once, O written once; an inference forward stores no log-sum-exp); the bound is
        # whichever needs longer at peak
        attn_flops = W.attention_fwd_flops(lengths, m, d, full_history=bool(vflags & 1))
        attn_bytes = T * 3 * d * es + T * d * es
        peak_f = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        if attn_bytes / (PEAK_HBM_GBS * 1e9) >= attn_flops / (peak_f * 1e12):
            work["attn_fwd"] = ("hbm", attn_bytes, "GB/s")
        else:
            work["attn_fwd"] = ("mfma", attn_flops, "TFLOP/s")
        work["qkv_gemm"] = ("hbm", (T * d + 3 * d * d + T * 3 * d) * es, "GB/s")
        work["out_gemm"] = ("hbm", (T * d + d * d + T * d) * es, "GB/s")
    # counter traffic was taken on the workload's own id distribution
    traffic = load_traffic(cfg.name) if args.item_dist is None else {}

    def rate(name, t_ms):
        if name not in work:
            return {"time_us": round(t_ms * 1e3, 2)}
        bound, amount, unit = work[name]
        if unit == "GB/s":
            achieved, peak = amount / (t_ms * 1e-3) / 1e9, PEAK_HBM_GBS
        else:
            achieved = amount / (t_ms * 1e-3) / 1e12
            peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        return {"time_us": round(t_ms * 1e3, 2), "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "algorithmic": int(amount),
                "traffic": traffic.get(name)}
    kernels = {name: rate(name, t_ms) for name, t_ms in per.items()}
    dominant = max((n for n in kernels if "bound" in kernels[n]), key=lambda n: kernels[n]["time_us"])

    # timed pass: exactly --steps steps between two device synchronisations, with one event
    # pair around the dominant kernel (on the stream it runs on) and none between the others
    events = [mk(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], only=dominant)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    t_dom = float(np.mean([events[k][0].elapsed_time(events[k][1]) for k in range(args.steps)]))
    kernels[dominant] = rate(dominant, t_dom)
    kernels[dominant]["timed_in"] = "timed pass"
    log(f"{ms:.4f} ms/step; {dominant} {t_dom * 1e3:.1f} us in the timed pass")
    kd = kernels[dominant]
    roofline = {"kernel": dominant, "bound": kd["bound"], "achieved": kd["achieved"], "peak": kd["peak"],
                "unit": kd["unit"], "frac": kd["frac"], "traffic": kd["traffic"]}

    cpu = None
    if args.cpu_seconds > 0:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(cfg, batch, tables, weights, args.cpu_seconds, (vflags, vedges))
        log(f"CPU oracle: {cpu['value']:.1f} candidates/s on {cpu['cores']} threads")

    cands = inp.B * m
    out = {
        "metric": METRIC,
        "value": round(cands / (ms * 1e-3), 1),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; Zipf(1.1) item ids, jagged histories, runs of 1-4 actions per request)",
        "config": {"workload": cfg.name, "users": inp.B, "candidates_per_user": m,
                   "history": f"U[{cfg.hist_min},{cfg.hist_max}]", "rows": T, "d": d, "heads": H,
                   "layers": cfg.layers, "block": cfg.block, "attn_variant": args.attn_variant},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernel_timing": "each kernel: its own pass of --steps steps with one event pair around it; the "
                         "dominant kernel: the event pair in the timed pass",
    }
    if attn_flops is not None:
        peak_f = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        tf = attn_flops / (kernels["attn_fwd"]["time_us"] * 1e-6) / 1e12
        kernels["attn_fwd"]["tflops"] = round(tf, 2)
        kernels["attn_fwd"]["flops"] = int(attn_flops)
        out["attn_mfma_util_pct"] = round(100 * tf / peak_f, 2)
    if decomposed:
        # sum-of-kernels roofline: each kernel at its own bound (bytes at 8 TB/s or flops at
        # the dense peak), against the measured step
        floor_us = sum((amount / (PEAK_HBM_GBS * 1e9) if unit == "GB/s" else
                        amount / ((PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS) * 1e12)) * 1e6
                       for _, (bound, amount, unit) in work.items())
        out["step_roofline_us"] = round(floor_us, 2)
        out["step_roofline_frac"] = round(floor_us / (ms * 1e3), 4)
    out["gather_gbps"] = kernels["embed_sum"]["achieved"]
    # the same launch against its logical bytes (five table rows read and one row written
    # per token): repeated rows that hit in cache count every time
    logical = W.gather_logical_bytes(T, d, es, idx_bytes)
    kernels["embed_sum"]["logical_bytes"] = int(logical)
    out["gather_logical_gbps"] = round(logical / (kernels["embed_sum"]["time_us"] * 1e-6) / 1e9, 2)
    if kernels["embed_sum"].get("traffic"):
        out["gather_dram_gbps"] = round(kernels["embed_sum"]["traffic"] / (kernels["embed_sum"]["time_us"] * 1e-6)
                                        / 1e9, 2)
    out["config"]["item_dist"] = cfg.item_dist
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
