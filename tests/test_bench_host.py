"""Host logic of bench.py's counter bookkeeping (--write-traffic): the dispatches before the
calibration copy map onto the step's units in order, a unit of several dispatches sums
their counters, and each counter is scaled by what it reads for the copy.  No GPU: the
counter files are written here in rocprofv3's CSV layout."""
import csv
import json

import bench

K_GEMM = "void genrank::(anonymous namespace)::gemm_nt_bf16_big_kernel<0, false>(genrank::(anonymous namespace)::GemmArgs)"
K_DQ = "void genrank::(anonymous namespace)::attn_bwd_dq_kernel<0>(genrank::(anonymous namespace)::BwdMArgs)"
K_DKV = "void genrank::(anonymous namespace)::attn_bwd_dkv_kernel<0>(genrank::(anonymous namespace)::BwdMArgs)"
K_COPY = "void at::native::copyBuffer(...)"


def _counters(d, counter, rows):
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, values) in enumerate(rows):
            for name, v in zip(counter, values):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": v})


def test_write_traffic_groups_and_scales(tmp_path):
    order = tmp_path / "order.json"
    order.write_text(json.dumps({"workload": "w", "copy_mib": 256,
                                 "units": [["L0.qkv", "qkv"], ["attn_bwd", "attn_bwd", 2]]}))
    # a warm-up dispatch, the units (one GEMM, then dQ + dK/dV), then the 256 MiB copy
    _counters(tmp_path / "f", ["FETCH_SIZE"], [(K_GEMM, [999.0]), (K_GEMM, [100.0]), (K_DQ, [30.0]),
                                               (K_DKV, [12.0]), (K_COPY, [131072.0])])
    _counters(tmp_path / "w", ["WRITE_SIZE"], [(K_GEMM, [999.0]), (K_GEMM, [50.0]), (K_DQ, [4.0]),
                                               (K_DKV, [6.0]), (K_COPY, [262144.0])])
    _counters(tmp_path / "m", ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
              [(K_GEMM, [1.0, 1.0]), (K_GEMM, [1024.0 * 16, 8.0 * 32]), (K_DQ, [1024.0 * 2, 8.0 * 10]),
               (K_DKV, [1024.0 * 6, 8.0 * 30]), (K_COPY, [0.0, 8.0])])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(order), str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "m"), out_path=str(out))
    rec = json.loads(out.read_text())["w"]
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    q, b = rec["qkv"], rec["attn_bwd"]
    assert q["kernel"] == "gemm_nt_bf16_big_kernel<0, false>"
    assert (q["fetch_bytes"], q["write_bytes"]) == (100 * 1024 * 2, 50 * 1024)
    assert b["kernel"] == "attn_bwd_dq_kernel<0> + attn_bwd_dkv_kernel<0>"
    assert (b["fetch_bytes"], b["write_bytes"]) == (42 * 1024 * 2, 10 * 1024)
    assert (b["fetch_kib_raw"], b["write_kib_raw"]) == (42, 10)
    # MFMA busy: busy cycles over 1024 SIMDs x the launch's cycles (GRBM over 8 XCDs), summed
    # over the unit's dispatches: (2 + 6) * 1024 / (1024 * (10 + 30)) = 20%
    assert q["mfma_busy_pct"] == 50.0
    assert b["mfma_busy_pct"] == 20.0
    # records carry the hash of their kernel's source, which load_traffic compares
    assert b["source_sha"] == bench.source_sha("attn_bwd.hip")
