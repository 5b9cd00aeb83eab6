"""bench.py's host-side bookkeeping, on synthetic counter files (no GPU): the HBM traffic
record scales FETCH_SIZE / WRITE_SIZE by the calibration kernel's readings, sums only the
grouped-GEMM kernels, and is ignored once the kernel source no longer matches it."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(d, sub, rows, counter):
    os.makedirs(os.path.join(d, sub), exist_ok=True)
    with open(os.path.join(d, sub, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_traffic_record_scaling_and_source_guard(tmp_path, monkeypatch):
    d = str(tmp_path / "prof")
    n = 1 << 30
    # the calibration kernel reads 6 GiB and writes 2 GiB; FETCH_SIZE reports half of it
    _csv(d, "cal_fetch", [("moe::(anonymous namespace)::residual_kernel(...)", 3 * n / 1024)], "FETCH_SIZE")
    _csv(d, "cal_write", [("moe::(anonymous namespace)::residual_kernel(...)", 2 * n / 1024)], "WRITE_SIZE")
    gemm = "void moe::(anonymous namespace)::gemm_stream_kernel<true, true, 4, 4>(...)"
    plan = "moe::(anonymous namespace)::plan_kernel(...)"
    other = "moe::(anonymous namespace)::copy_kernel(...)"
    # two dispatches of the GEMM (mean 1000 KiB fetched), one plan, and a kernel that must not count
    _csv(d, "fetch_w", [(gemm, 900.0), (gemm, 1100.0), (plan, 2.0), (other, 1e9)], "FETCH_SIZE")
    _csv(d, "write_w", [(gemm, 50.0), (gemm, 50.0), (plan, 1.0), (other, 1e9)], "WRITE_SIZE")
    out = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out)
    rec = bench.write_traffic(d, ["w"])
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    w = rec["workloads"]["w"]
    assert w["read_bytes_per_call"] == round(1000 * 1024 * 2.0) + round(2 * 1024 * 2.0)
    assert w["write_bytes_per_call"] == 50 * 1024 + 1024
    assert w["hbm_bytes_per_call"] == w["read_bytes_per_call"] + w["write_bytes_per_call"]
    assert w["per_kernel_per_launch"]["gemm_stream_kernel<true, true, 4, 4>"]["dispatches"] == 2
    assert sorted(w["per_kernel_per_launch"]) == ["gemm_stream_kernel<true, true, 4, 4>", "plan_kernel"]
    assert json.load(open(out)) == rec
    # read back only while the kernel source is the one the counters were taken on
    assert bench.traffic_from_profiles("w") == w
    monkeypatch.setattr(bench, "_source_sha256", lambda: "0" * 64)
    assert bench.traffic_from_profiles("w") is None


def test_cpu_baseline_bulk_leg():
    """bench.py's cpu_baseline leg on the tiny fp32 layer: it runs the oracle's bulk float32
    path over the whole layer, reports the threads it used, and compares the output it is
    handed (here the float64 oracle's own) to its own result."""
    import numpy as np
    from grouped_gemm_weights_amd import synth
    from oracle import moe as O
    cfg = synth.config("tiny_fp32_t64")
    blocks = {e: b for e, b in enumerate(synth.pool_np(cfg, 0, range(cfg.E)))}
    ref = O.moe_layer(synth.activations(cfg), synth.logits(cfg), cfg.k, lambda e: blocks[e],
                      cfg.H, cfg.I, False)
    r = bench.cpu_baseline_bulk(cfg, blocks, ref["y"], 8)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] >= 1 and r["single_thread"]["value"] > 0
    assert r["gpu_vs_cpu_max_err_over_rms"] <= 1e-5
    assert set(r["tiny_fp32_t64"]) == {"all_threads", "single_thread"}


def test_cpu_baseline_sample_leg():
    """bench.py's sampled cpu_baseline leg of the prefill workloads, on the tiny fp32 layer:
    the oracle's grouped step over a few experts with all their rows, scaled to tokens/s by
    the share of assignments, compared with the y_perm rows it is handed (here the float64
    oracle's own)."""
    import numpy as np
    from grouped_gemm_weights_amd import synth
    from oracle import moe as O
    cfg = synth.config("tiny_fp32_t64")
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    ref = O.moe_layer(synth.activations(cfg), synth.logits(cfg), cfg.k, lambda e: blocks[e],
                      cfg.H, cfg.I, False)
    off, src_of = np.asarray(ref["offsets"]), np.asarray(ref["src_of"])
    pick = [1, 5, 6]
    rows = [np.arange(off[e], off[e + 1]) for e in pick]
    s = {"experts": pick, "n_active": cfg.E, "R": cfg.T * cfg.k,
         "xp": np.concatenate([synth.activations(cfg)[src_of[r] // cfg.k] for r in rows]),
         "off": np.concatenate([[0], np.cumsum([len(r) for r in rows])]),
         "blocks": [blocks[e] for e in pick],
         "yp": np.concatenate([np.asarray(ref["y_perm"])[r] for r in rows])}
    r = bench.cpu_baseline_sample(cfg, s)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["experts"] == pick and r["cores"] >= 1
    assert r["gpu_vs_cpu_max_err_over_rms"] <= 1e-5
    assert f"({int(s['off'][-1])} of {cfg.T * cfg.k} assignments)" in r["sample"]
