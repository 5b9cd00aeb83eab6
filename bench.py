#!/usr/bin/env python3
"""Throughput of the DWDP-style MoE layer forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
with the weight pools and inputs already resident in HBM:

    route -> permute (counts, offsets, permutation, row gather)
    -> copy stream (after an event on the permute): merge the local experts
       into the merged buffer half and pull the routed remote experts from the
       stand-in peer pool, the routed set read from the counts on the device
       (--remote routed reads the counts back to the host and pulls that set)
    -> compute stream waits for the copies -> grouped SwiGLU GEMM -> combine

Steps alternate between the two halves of the double buffer.  The default
workload is the DeepSeek-R1-shaped decode step (64 tokens, hidden 7168,
256 experts with SwiGLU intermediate 2048, top-8, 64 local / 192 remote).

Prints ONE JSON line: tokens/s of the whole step, the roofline of the
dominant kernel (the grouped SwiGLU GEMM, timed with HIP events on its own
stream inside the timed region), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="r1_decode_t64")
    p.add_argument("--remote", choices=["device", "routed", "all"], default="device",
                   help="prefetch only the routed remote experts (device: picked on the device "
                        "from the counts, nothing read back; routed: after a count read-back), "
                        "or the whole remote share")
    p.add_argument("--pipeline-graph-steps", type=int, default=3,
                   help="pipelines: also replay the pass captured into one HIP graph this many "
                        "times (0: skip); reported beside the value, not as it")
    p.add_argument("--graph-steps", type=int, default=20,
                   help="headline with --remote device: also replay the step captured into a HIP "
                        "graph this many times (0: skip); reported beside the value, not as it")
    p.add_argument("--cpu-sample-experts", type=int, default=32,
                   help="prefill workloads: time the oracle's grouped step on this many of the "
                        "layer's active experts (0: skip)")
    p.add_argument("--copy-mode", choices=["sdma", "any", "kernel"], default="kernel",
                   help="any: hipMemcpyDefault (the runtime's copy path); sdma: the no-compute-unit "
                        "copy kind; kernel: the library's copy kernel on --copy-blocks workgroups")
    p.add_argument("--copy-blocks", type=int, default=0,
                   help="workgroups of the copy kernel (--copy-mode kernel; 0: no limit)")
    p.add_argument("--alt-steps", type=int, default=5,
                   help="also time this many steps with the other copy mode (0: skip)")
    p.add_argument("--chunks", type=int, default=0,
                   help="split the remote fetch into this many chunks, each with its own ready "
                        "event, and run the grouped GEMM per chunk as it lands (0: one fetch, one GEMM)")
    p.add_argument("--gather", choices=["separate", "fused"], default="fused",
                   help="separate: moe_permute writes x_perm; fused: the grouped GEMM gathers its rows "
                        "from x on load (moe_grouped_swiglu_gathered)")
    p.add_argument("--combine", choices=["separate", "epilogue"], default="separate",
                   help="separate: grouped GEMM writes y_perm, moe_combine sums it; epilogue: the "
                        "down GEMM adds its weighted rows into y (moe_grouped_swiglu_combine)")
    p.add_argument("--merge", choices=["copy", "stitched"], default="stitched",
                   help="copy the local experts into each merged half, or stitch the local "
                        "block into the half's virtual range so the merge copies nothing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-single-thread-tokens", type=int, default=8,
                   help="tokens of the layer also run through the CPU bulk path with one BLAS "
                        "thread (0: skip)")
    p.add_argument("--workloads",
                   default="r1_prefill_t8192_zipf,r1_prefill_t16384,r1_pipeline_6x4096,"
                           "r1_decode_t64_host_pool",
                   help="other workloads timed in the same run and reported under 'workloads' "
                        "('none': only the headline); a name ending in _host_pool is that "
                        "workload with its remote pool in pinned host memory")
    p.add_argument("--remote-pool", choices=["device", "host"], default="device",
                   help="where the remote experts live: a device pool, or pinned host memory "
                        "(pulled over PCIe by the runtime copy)")
    p.add_argument("--sdma-experts", type=int, default=0,
                   help="pipelines: pull this many remote experts per layer as no-CU copies on a "
                        "second copy stream, beside the rest (0: one copy stream)")
    p.add_argument("--pipeline-chunks", type=int, default=1,
                   help="pipelines: cut the main pull into this many expert-aligned chunks, each "
                        "with its own ready event; the grouped GEMM runs per chunk as it lands")
    p.add_argument("--workload-steps", type=int, default=10)
    p.add_argument("--no-library-baseline", dest="library_baseline", action="store_false",
                   help="skip timing the vendor BLAS on the same per-expert GEMMs")
    p.add_argument("--pipeline-steps", type=int, default=3)
    p.add_argument("--calibrate", action="store_true",
                   help="run only a plain streaming kernel of known size (moe_residual_add over "
                        "1 GiB elements), the reference for scaling the HBM byte counters")
    p.add_argument("--write-traffic", metavar="PROF_DIR",
                   help="no GPU work: turn rocprofv3 FETCH_SIZE / WRITE_SIZE csv runs under "
                        "PROF_DIR (fetch_<config>, write_<config>, cal_fetch, cal_write) for the "
                        "configs given with --traffic-configs into profiles/grouped_swiglu_traffic.json")
    p.add_argument("--traffic-configs", default="r1_decode_t64")
    return p.parse_args()


def cpu_baseline_bulk(cfg, blocks, y_gpu, single_thread_tokens=0):
    """The oracle's bulk path over the whole layer: route, stable permutation, gather, then per
    expert (one expert's weights decoded at a time, from host copies of the bytes the GPU read)
    float32 products with h rounded to bf16 as the GPU stores it, and the float32 combine.
    The GPU's output of the same step is compared with it (max|err|/RMS)."""
    import numpy as np
    from oracle import moe as O
    from grouped_gemm_weights_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = synth.activations(cfg)
    logits = synth.logits(cfg)
    rh = cfg.dtype == "bf16"
    t0 = time.perf_counter()
    res = O.moe_layer(x, logits, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, round_h=rh,
                      dtype=np.float32)
    dt = time.perf_counter() - t0
    ref = res["y"].astype(np.float64)
    err = float(np.max(np.abs(np.asarray(y_gpu, np.float64) - ref)) / np.sqrt(np.mean(ref ** 2)))
    out = {"value": round(cfg.T / dt, 4), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"the whole {cfg.T}-token layer, route to combine, through the oracle's bulk "
                     f"float32 path ({len(blocks)} experts decoded one at a time), {dt:.1f} s",
           "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
           "gpu_vs_cpu_max_err_over_rms": round(err, 6)}
    if single_thread_tokens > 0:
        from threadpoolctl import threadpool_limits
        n = min(single_thread_tokens, cfg.T)
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            O.moe_layer(x[:n], logits[:n], cfg.k, lambda e: blocks[e], cfg.H, cfg.I, round_h=rh,
                        dtype=np.float32)
            d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": round(n / d1, 4), "unit": "tokens/s",
                                "sample": f"the same path on the first {n} tokens, one BLAS "
                                          f"thread, {d1:.1f} s"}
    # the tiny fp32 layer (64 tokens, 8 experts) through the same path, whole, at full and
    # at one BLAS thread (its weights are drawn on the host)
    from threadpoolctl import threadpool_limits
    tc = synth.config("tiny_fp32_t64")
    tb = synth.pool_np(tc, 0, range(tc.E))
    tx, tl = synth.activations(tc), synth.logits(tc)
    tiny = {}
    for name, lim in (("all_threads", None), ("single_thread", 1)):
        with threadpool_limits(limits=lim):
            reps, t2 = 0, time.perf_counter()
            while True:
                O.moe_layer(tx, tl, tc.k, lambda e: tb[e], tc.H, tc.I, round_h=False,
                            dtype=np.float32)
                reps += 1
                if time.perf_counter() - t2 > 0.5:
                    break
            d2 = (time.perf_counter() - t2) / reps
        tiny[name] = {"value": round(tc.T / d2, 1), "unit": "tokens/s", "ms": round(d2 * 1e3, 3)}
    out["tiny_fp32_t64"] = tiny
    return out


def cpu_baseline_sample(cfg, s):
    """The oracle's bulk float32 grouped SwiGLU step on a seeded sample of a prefill layer's
    active experts, each with all its rows: the step that holds nearly all of the layer's
    work, on a sample, since the oracle decodes every expert's weights from bf16 one at a time
    (a whole 256-expert layer is about a minute of CPU).  tokens/s = T * (sample rows / R) /
    time.  The GPU's y_perm rows of the same experts are compared with it (max|err|/RMS)."""
    import numpy as np
    from oracle import moe as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    blocks = s["blocks"]
    t0 = time.perf_counter()
    y = O.grouped_swiglu(s["xp"], s["off"], lambda i: blocks[i], cfg.H, cfg.I,
                         round_h=cfg.dtype == "bf16", dtype=np.float32)
    dt = time.perf_counter() - t0
    ref = y.astype(np.float64)
    err = float(np.max(np.abs(np.asarray(s["yp"], np.float64) - ref)) / np.sqrt(np.mean(ref ** 2)))
    rows = int(s["off"][-1])
    return {"value": round(cfg.T * rows / s["R"] / dt, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(blocks)} of the layer's {s['n_active']} active experts (seeded), each "
                      f"with all its rows ({rows} of {s['R']} assignments), through the oracle's "
                      f"bulk float32 grouped SwiGLU step; tokens/s = T * rows / R / time; "
                      f"{dt:.1f} s",
            "experts": s["experts"], "gpu_vs_cpu_max_err_over_rms": round(err, 6)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def input_digests(cfg, local, remote):
    """SHA-256 of the seeded inputs: logits, activations and a strided sample of each weight
    pool (every 2^20-th element), so two runs can be shown to have used the same data."""
    from grouped_gemm_weights_amd import synth
    d = {"logits": synth.digest(synth.logits(cfg)), "x": synth.digest(synth.activations(cfg))}
    for name, pool in (("local_pool_sample", local), ("remote_pool_sample", remote)):
        if pool is not None and pool.numel() > 0:
            d[name] = synth.digest(pool.view(-1)[::1 << 20])
    return d


def bench_pipeline(args, cfg, dev, copy_mode):
    """The multi-layer pipeline: prefetch of layer l+1 on the copy stream hidden behind layer
    l's MoE block and layer l+1's dense stand-in block; hidden fraction and per-layer latency."""
    import numpy as np
    import torch
    from grouped_gemm_weights_amd import binding as B
    from grouped_gemm_weights_amd import synth
    from grouped_gemm_weights_amd.pipeline import MoEPipeline

    P = MoEPipeline(cfg, device=dev, copy_mode=copy_mode, stitched=args.merge == "stitched",
                    fused_gather=args.gather == "fused", sdma_experts=args.sdma_experts,
                    chunks=args.pipeline_chunks)
    split = P.split
    n = cfg.layers
    keys = ("c0", "c1", "wait0", "wait1", "d0", "m1", "g1")
    mk = lambda: {k: [B.moe_event_create(True) for _ in range(n)] for k in keys}
    for _ in range(args.warmup):
        P.forward()
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        P.forward(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert P.L.read_status() == 0, "device status set during the benchmark"
    el = B.moe_event_elapsed_ms
    P_l, stall, Lat, comp_pipe, gemm = [], [], [], [], []
    for ev in evs:
        for l in range(n):
            P_l.append(el(ev["c0"][l], ev["c1"][l]))
            stall.append(el(ev["wait0"][l], ev["wait1"][l]))
            comp_pipe.append(el(ev["d0"][l], ev["m1"][l]) - stall[-1])
            # split pull: the GEMM runs as expert ranges between waits, timed from the first
            # wait to the last range's end (waits included: an upper bound)
            gemm.append(el(ev["wait0" if split else "wait1"][l], ev["g1"][l]))
            if l > 0:
                Lat.append(el(ev["m1"][l - 1], ev["m1"][l]))
    sev = mk()
    P.forward_serial(sev)
    torch.cuda.synchronize()
    C_alone = [el(sev["d0"][l], sev["m1"][l]) for l in range(n)]
    P_alone = [el(sev["c0"][l], sev["c1"][l]) for l in range(n)]
    copy_bytes = (cfg.E - (cfg.n_local if P.stitched else 0)) * synth.expert_block_bytes(cfg)
    graph_rec = None
    gsteps = getattr(args, "pipeline_graph_steps", 0)
    if gsteps > 0 and not split:
        # the pipelined pass captured into one HIP graph and replayed (not the reported value):
        # each replay must reproduce the eager pass's final residual stream bit for bit
        P.forward()
        torch.cuda.synchronize()
        x_eager = P.x.clone()
        g = P.capture()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(P.x, x_eager))
        tg = time.perf_counter()
        for _ in range(gsteps):
            g.replay()
        torch.cuda.synchronize()
        g_s = (time.perf_counter() - tg) / gsteps
        same = same and bool(torch.equal(P.x, x_eager))
        assert P.L.read_status() == 0, "device status set during the graph replays"
        graph_rec = {"passes": gsteps, "ms_per_pass": round(g_s * 1e3, 3),
                     "tokens_per_s": round(cfg.T / g_s, 2), "x_bit_equal_to_eager": same}
        del g
    P.close()
    for e in [e for ev in evs + [sev] for lst in ev.values() for e in lst]:
        B.moe_event_destroy(e)
    del P
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    mean = lambda v: float(np.mean(v))
    # with a split pull the compute stream runs expert ranges between its waits, so the time
    # around the waits is not a stall: no hidden fraction then, the latency figures stand
    H = None if split else 1.0 - sum(stall) / sum(P_l)
    eb = synth.expert_block_bytes(cfg)
    R = cfg.T * cfg.k
    gemm_ms = mean(gemm)
    alg_bytes = cfg.E * eb + R * cfg.H * 6
    alg_flop = 6.0 * cfg.H * cfg.I * R
    gbps = alg_bytes / (gemm_ms * 1e-3) / 1e9
    tflops = alg_flop / (gemm_ms * 1e-3) / 1e12
    if alg_flop / alg_bytes < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof.update({"traffic": None,
                 "kernel": "moe_grouped_swiglu, pipelined layers (with the copy running)" +
                           (", expert ranges as the pull lands, waits included" if split else ""),
                 "avg_ms": round(gemm_ms, 4), "alg_bytes": alg_bytes, "alg_flop": alg_flop,
                 "TFLOPs": round(tflops, 1), "GBps": round(gbps, 1)})
    return {
        "metric": "MoE layer tokens/s + grouped-GEMM % of HBM/MFMA roofline, R1 shape, 1 GPU",
        "value": round(cfg.T * args.steps / wall, 2), "unit": "tokens/s (through all layers)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "layers": n, "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "top_k": cfg.k,
                   "local_experts": cfg.n_local, "copy_engine": args.copy_mode,
                   "copy_blocks": args.copy_blocks if args.copy_mode == "kernel" else None,
                   "merge": args.merge, "gather": args.gather, "sdma_experts": args.sdma_experts,
                   "pull_chunks": args.pipeline_chunks, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "pipeline": {
            "prefetch_ms": round(mean(P_l), 3), "prefetch_alone_ms": round(mean(P_alone), 3),
            "copy_bytes": copy_bytes,
            "copy_GBps": round(copy_bytes / (mean(P_l) * 1e-3) / 1e9, 1),
            "stall_ms": None if split else round(mean(stall), 3),
            "hidden_fraction": None if H is None else round(H, 4),
            "compute_pipelined_ms": None if split else round(mean(comp_pipe), 3),
            "compute_alone_ms": round(mean(C_alone), 3),
            "contention_slowdown": None if split else round(mean(comp_pipe) / mean(C_alone), 3),
            "layer_latency_ms": round(mean(Lat), 3),
            "layer_latency_ms_median": round(float(np.median(Lat)), 3),
            "layer_latency_ms_min": round(float(np.min(Lat)), 3),
            "max_compute_prefetch_ms": round(max(mean(C_alone), mean(P_alone)), 3),
            "sum_compute_prefetch_ms": round(mean(C_alone) + mean(P_alone), 3),
            # how close the layer comes to max(C, P), the per-layer latency panel's ideal
            "latency_over_max_compute_prefetch": round(mean(Lat) / max(mean(C_alone), mean(P_alone)), 3),
            # share of the prefetch's own time that the overlap actually saves:
            # (C_alone + P_alone - L) / P_alone; 1 = fully hidden at no cost, 0 = serial
            "overlap_efficiency": round((mean(C_alone) + mean(P_alone) - mean(Lat)) / mean(P_alone), 3),
            # one GPU moves per layer the weights the GEMMs read, the dense block's weight and
            # the pull twice (a read and a write of the same HBM): its time at 8 TB/s
            "hbm_floor_ms": round((cfg.E * eb + cfg.H * cfg.H * 2 + 2 * copy_bytes) / HBM_PEAK_GBPS / 1e6, 3),
            "hidden_fraction_definition": "1 - stall/prefetch: time the compute stream waits for "
                                          "the copy, not the slowdown the copy causes",
        },
        "graph_replay": graph_rec,
    }


def calibrate():
    """A plain streaming kernel with known traffic: out = bf16(x + y) over n elements reads
    2n + 4n bytes and writes 2n bytes."""
    import torch
    from grouped_gemm_weights_amd import binding as B
    n = 1 << 30
    dev = torch.device("cuda:0")
    x = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(n, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        B.moe_residual_add(x, y, n, out, None)
    torch.cuda.synchronize()
    return {"kernel": "residual_kernel", "launches": 3, "read_bytes_per_launch": 6 * n,
            "write_bytes_per_launch": 2 * n}


GEMM_SOURCE = os.path.join(ROOT, "grouped_gemm_weights_amd", "csrc", "grouped_swiglu.hip")
# the short bench run the counter passes profile (one workload, nothing timed beside it)
PROFILE_ARGS = ("--config {cfg} --steps 2 --warmup 1 --workloads none --no-cpu-baseline "
                "--no-library-baseline --alt-steps 0 --graph-steps 0")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_swiglu_traffic.json")
# kernels of one moe_grouped_swiglu call
GROUPED_KERNELS = ("plan_kernel", "gemm_stream_kernel", "gemm_wide_kernel")


def _source_sha256():
    import hashlib
    return hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()


def traffic_from_profiles(workload):
    """HBM bytes per moe_grouped_swiglu call of `workload` measured with rocprofv3 counters, if
    they were taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_source_sha256") != _source_sha256():
        return None
    return rec.get("workloads", {}).get(workload)


def write_traffic(prof_dir, workloads):
    """Scale per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) by what the same counters read for the
    calibration kernel (6 GiB read, 2 GiB written per launch) and record the per-call HBM bytes
    of moe_grouped_swiglu for each workload."""
    import collections
    import csv

    def load(sub):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(prof_dir, sub, "run_counter_collection.csv"))):
            d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return d

    def mean(v):
        return sum(v) / len(v)

    n = 1 << 30
    cal_f = [v for k, v in load("cal_fetch").items() if "residual_kernel" in k][0]
    cal_w = [v for k, v in load("cal_write").items() if "residual_kernel" in k][0]
    fetch_scale = 6 * n / (mean(cal_f) * 1024)
    write_scale = 2 * n / (mean(cal_w) * 1024)
    rec = {
        "kernel_source_sha256": _source_sha256(),
        "calibration": {"kernel": "moe_residual_add over 2^30 elements (reads 6 GiB, writes 2 GiB)",
                        "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
        "workloads": {},
    }
    for cfg in workloads:
        f, w = load(f"fetch_{cfg}"), load(f"write_{cfg}")
        per = {}
        for k in f:
            if not any(s in k for s in GROUPED_KERNELS):
                continue
            short = k.replace("moe::(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            per[short] = {"read_bytes": round(mean(f[k]) * 1024 * fetch_scale),
                          "write_bytes": round(mean(w[k]) * 1024 * write_scale),
                          "dispatches": len(f[k])}
        rd = sum(v["read_bytes"] for v in per.values())
        wr = sum(v["write_bytes"] for v in per.values())
        rec["workloads"][cfg] = {
            "per_kernel_per_launch": per, "read_bytes_per_call": rd, "write_bytes_per_call": wr,
            "hbm_bytes_per_call": rd + wr,
            "commands": [
                f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch_{cfg} -o run -- "
                f"python3 bench.py {PROFILE_ARGS.format(cfg=cfg)}",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write_{cfg} -o run -- "
                f"python3 bench.py {PROFILE_ARGS.format(cfg=cfg)}",
            ],
        }
    rec["calibration"]["commands"] = [
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/cal_fetch -o run -- python3 bench.py --calibrate",
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/cal_write -o run -- python3 bench.py --calibrate",
    ]
    rec["output_dir"] = "$OUT: the directory the runs above wrote to (read by --write-traffic)"
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    return rec


def main():
    args = parse()
    if args.write_traffic:
        rec = write_traffic(args.write_traffic, args.traffic_configs.split(","))
        print(json.dumps(rec, indent=1))
        return
    if args.calibrate:
        print(json.dumps(calibrate()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path, every "
              f"figure is one GPU's share (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from grouped_gemm_weights_amd import binding as B
    from grouped_gemm_weights_amd import synth

    cfg = synth.config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_mode = {"sdma": B.MOE_COPY_SDMA, "any": B.MOE_COPY_ANY,
                 "kernel": B.copy_kernel_on(args.copy_blocks)}[args.copy_mode]
    if cfg.layers != 1:
        print(json.dumps(bench_pipeline(args, cfg, dev, copy_mode)), flush=True)
        return
    host_blocks = {}
    result = bench_layer(args, cfg, dev, copy_mode, args.steps, args.warmup, args.alt_steps,
                         headline=True, host_blocks=host_blocks,
                         remote_on_host=args.remote_pool == "host", graph_steps=args.graph_steps)
    # the other R1 workloads in the same run, each timed as above (default options), so the
    # prefill MFMA fractions and the pipeline's overlap figures sit beside the headline
    names = [w for w in args.workloads.split(",") if w and w != "none"]
    if names:
        wl = {}
        for name in names:
            host_pool = name.endswith("_host_pool")
            c = synth.config(name[: -len("_host_pool")] if host_pool else name)
            t0 = time.perf_counter()
            if host_pool:
                # the offload variant: every pull crosses PCIe, so a few steps suffice; a host
                # pool is pulled by the copy engine after the count read-back
                ha = argparse.Namespace(**vars(args))
                if ha.remote == "device":
                    ha.remote = "routed"
                r = bench_layer(ha, c, dev, copy_mode, 3, 1, 0, remote_on_host=True)
                wl[name] = layer_summary(r)
            elif c.layers == 1:
                ns = 0 if args.no_cpu_baseline else args.cpu_sample_experts
                r = bench_layer(args, c, dev, copy_mode, args.workload_steps, 2, 0, cpu_sample=ns)
                wl[name] = layer_summary(r)
                if "_cpu_sample" in r:
                    wl[name]["cpu_baseline"] = cpu_baseline_sample(c, r.pop("_cpu_sample"))
            else:
                pa = argparse.Namespace(**vars(args))
                pa.steps, pa.warmup = args.pipeline_steps, 1
                wl[name] = pipeline_summary(bench_pipeline(pa, c, dev, copy_mode))
            wl[name]["bench_wall_s"] = round(time.perf_counter() - t0, 1)
            print(f"[bench] {name} done in {wl[name]['bench_wall_s']} s", file=sys.stderr, flush=True)
        result["workloads"] = wl
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_bulk(cfg, host_blocks, result.pop("_y"),
                                                   args.cpu_single_thread_tokens)
    result.pop("_y", None)
    print(json.dumps(result), flush=True)


def library_baseline(L, cfg, reps=3):
    """The same grouped GEMM work done by the vendor BLAS (hipBLASLt through torch's
    F.linear), one call per active expert and projection -- [rows, H] x [2I, H]^T for gate
    and up together, then [rows, I] x [H, I]^T -- on the weight bytes of the layer's pools,
    SiLU left out.  Context for the grouped kernel's time, not part of the path."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    H, I, k = cfg.H, cfg.I, cfg.k
    counts = L.counts.cpu().numpy()
    offs = L.offsets.cpu().numpy()
    xp = L.x.index_select(0, (L.src_of // k).long())          # x_perm, built outside the clock
    hs = torch.empty((L.R, I), dtype=xp.dtype, device=xp.device)
    experts = [int(e) for e in np.nonzero(counts)[0]]
    mats = []
    for e in experts:
        blk = L.expert_block(e)
        mats.append((int(offs[e]), int(offs[e + 1]), blk[: 2 * H * I].view(2 * I, H),
                     blk[2 * H * I:].view(H, I)))
    torch.cuda.synchronize()

    def run():
        for lo, hi, wgu, wd in mats:
            F.linear(xp[lo:hi], wgu)
            F.linear(hs[lo:hi], wd)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    flop = 6.0 * H * I * L.R
    del xp, hs, mats
    return {"kind": "hipBLASLt via torch F.linear, one call per active expert and projection "
                    "(gate and up as one [2I, H] matrix; SiLU left out)",
            "calls": 2 * len(experts), "ms": round(ms, 3),
            "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1)}


def layer_summary(r):
    """The figures of a single-layer record that matter beside the headline."""
    keep = ("value", "unit", "ms_per_step", "roofline", "breakdown_ms", "timing", "copy",
            "active_experts", "gemm_TFLOPs", "hbm_frac", "mfma_frac", "library_baseline")
    out = {k: r[k] for k in keep if k in r}
    out["config"] = {k: r["config"][k] for k in ("tokens", "remote_fetch", "merge", "gather",
                                                  "copy_engine", "combine")}
    return out


def pipeline_summary(r):
    out = {"value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
           "steps": r["steps"], "roofline": r["roofline"]}
    out.update(r["pipeline"])
    if r.get("graph_replay") is not None:
        out["graph_replay"] = r["graph_replay"]
    out["config"] = {k: r["config"][k] for k in ("layers", "tokens", "merge", "gather",
                                                  "copy_engine", "sdma_experts", "pull_chunks")}
    return out


def bench_layer(args, cfg, dev, copy_mode, steps, warmup, alt_steps, headline=False,
                host_blocks=None, remote_on_host=False, graph_steps=0, cpu_sample=0):
    """One MoE layer step timed over ``steps`` steps; returns its record.  With ``headline``
    the record also carries the input digests and the layer output (for the CPU comparison),
    and host copies of the routed experts' blocks are left in ``host_blocks``.  With
    ``cpu_sample`` > 0 it carries, under ``_cpu_sample``, a seeded sample of that many active
    experts: their gathered rows, weight blocks and the GPU's y_perm rows (taken after the
    timed region)."""
    import numpy as np
    import torch
    from grouped_gemm_weights_amd import binding as B
    from grouped_gemm_weights_amd import synth
    from grouped_gemm_weights_amd.layer import MoELayer, block_to_numpy

    comb = args.combine == "epilogue"
    L = MoELayer(cfg, device=dev, copy_mode=copy_mode, stitched=args.merge == "stitched",
                 fused_gather=args.gather == "fused", combine_in_epilogue=comb)
    local = synth.pool_torch(cfg, 0, 0, cfg.n_local, dev)
    remote = synth.pool_torch(cfg, 0, cfg.n_local, cfg.E - cfg.n_local, dev)
    if remote_on_host:
        host = torch.empty(remote.shape, dtype=remote.dtype, pin_memory=True)
        host.copy_(remote)
        del remote
        torch.cuda.empty_cache()
        remote = host
    L.set_pools(local, remote)
    L.set_inputs(synth.activations(cfg), synth.logits(cfg))
    cs, ps = L.compute_stream, L.copy_stream

    nev = steps
    mk = lambda: [B.moe_event_create(True) for _ in range(nev)]
    ev = {k: mk() for k in ("start", "rp_end", "gemm0", "gemm1", "end", "copy0", "copy1")}
    nch = max(0, args.chunks)
    on_device = args.remote == "device"
    if on_device and nch > 0:
        raise SystemExit("--remote device is not chunked")
    if on_device:
        alt_steps = 0              # the device-routed pull always runs on the copy kernel
    gev = [{"g0": [B.moe_event_create(True) for _ in range(nch + 1)],
            "g1": [B.moe_event_create(True) for _ in range(nch + 1)]} for _ in range(nev)]

    def step(i, timed):
        h = i % 2
        if timed:
            B.moe_event_record(ev["start"][i], cs)
        L.route_permute()
        if timed:
            B.moe_event_record(ev["rp_end"][i], cs)
        if on_device:
            ids = None
            # the copy stream's wait for the permute, ahead of its start event, so the copy's
            # time counts from the routing being known (the host does not wait here)
            B.moe_event_record(L.counts_ready, cs)
            B.moe_stream_wait_event(ps, L.counts_ready)
        else:
            ids = L.routed_ids() if args.remote == "routed" else list(range(cfg.E))
        if timed:
            B.moe_event_record(ev["copy0"][i], ps)
        if nch > 0:
            L.forward_chunked(h, ids, nch, gev[i] if timed else None)
            if timed:
                B.moe_event_record(ev["copy1"][i], ps)
                B.moe_event_record(ev["end"][i], cs)
            return ids
        if on_device:
            L.fill_half_routed_on_device(h)
        else:
            L.fill_half(h, ids)
        if timed:
            B.moe_event_record(ev["copy1"][i], ps)
        B.moe_stream_wait_event(cs, L.ready[h])
        if timed:
            B.moe_event_record(ev["gemm0"][i], cs)
        if comb:
            L.grouped_combine(L.wbufs[h])
        else:
            L.grouped(L.wbufs[h])
        if timed:
            B.moe_event_record(ev["gemm1"][i], cs)
        if not comb:
            B.moe_combine(L.y_perm, L.row_of, L.topk_w, cfg.T, cfg.k, cfg.H, L.y, cs)
        B.moe_event_record(L.free[h], cs)
        if timed:
            B.moe_event_record(ev["end"][i], cs)
        return ids

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ids = step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert L.read_status() == 0, "device status set during the benchmark"
    alt = None
    if alt_steps > 0:
        # the same step with the other copy path, for comparison (not the reported value)
        alt_name = "sdma" if args.copy_mode == "any" else "any"
        L.copy_mode = B.MOE_COPY_SDMA if alt_name == "sdma" else B.MOE_COPY_ANY
        for i in range(2):
            step(i, False)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for i in range(alt_steps):
            step(i, False)
        torch.cuda.synchronize()
        alt_s = (time.perf_counter() - ta) / alt_steps
        alt = {"copy_engine": alt_name,
               "ms_per_step": round(alt_s * 1e3, 3), "tokens_per_s": round(cfg.T / alt_s, 1)}
        L.copy_mode = copy_mode

    graph_rec = None
    if on_device and graph_steps > 0:
        # the same step captured into one HIP graph per half and replayed (not the reported
        # value): the replays must reproduce the eager step's y bit for bit
        y_eager = L.y.clone()
        graphs = [L.capture_step(h) for h in range(2)]
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(L.y, y_eager))
        tg = time.perf_counter()
        for i in range(graph_steps):
            graphs[i % 2].replay()
        torch.cuda.synchronize()
        g_s = (time.perf_counter() - tg) / graph_steps
        same = same and bool(torch.equal(L.y, y_eager))
        assert L.read_status() == 0, "device status set during the graph replays"
        graph_rec = {"steps": graph_steps, "ms_per_step": round(g_s * 1e3, 4),
                     "tokens_per_s": round(cfg.T / g_s, 1), "y_bit_equal_to_eager": same}
        del graphs

    el = lambda a, b: float(np.mean([B.moe_event_elapsed_ms(ev[a][i], ev[b][i]) for i in range(nev)]))
    if nch > 0:
        n_calls = nch + 1
        gemm_ms = float(np.mean([sum(B.moe_event_elapsed_ms(g["g0"][c], g["g1"][c]) for c in range(n_calls))
                                 for g in gev]))
        combine_ms = float(np.mean([B.moe_event_elapsed_ms(g["g1"][n_calls - 1], ev["end"][i])
                                    for i, g in enumerate(gev)]))
    else:
        gemm_ms = el("gemm0", "gemm1")
        combine_ms = el("gemm1", "end")
    rp_ms = el("start", "rp_end")
    copy_ms = el("copy0", "copy1")
    layer_ms = el("start", "end")
    per_step = lambda a, b: [B.moe_event_elapsed_ms(ev[a][i], ev[b][i]) for i in range(nev)]
    layer_v = per_step("start", "end")
    timing = {"layer_ms_median": round(float(np.median(layer_v)), 4),
              "layer_ms_min": round(float(np.min(layer_v)), 4)}
    if nch == 0:
        gemm_v = per_step("gemm0", "gemm1")
        timing.update({"grouped_swiglu_ms_median": round(float(np.median(gemm_v)), 4),
                       "grouped_swiglu_ms_min": round(float(np.min(gemm_v)), 4)})
    for lst in list(ev.values()) + [l for g in gev for l in g.values()]:
        for e in lst:
            B.moe_event_destroy(e)

    counts = L.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    if ids is None:                 # the device-routed set: every local expert and the routed rest
        ids = list(range(cfg.n_local)) + [e for e in range(cfg.n_local, cfg.E) if counts[e] > 0]
    eb = synth.expert_block_bytes(cfg)
    R = cfg.T * cfg.k
    # weights read + x_perm + y_perm; with the combine in the epilogue: + x rows read through
    # src_of and y accumulated in place (T rows of H floats)
    alg_bytes = n_active * eb + R * cfg.H * 2 + (cfg.T * cfg.H * 4 if comb else R * cfg.H * 4)
    alg_flop = 6.0 * cfg.H * cfg.I * R
    copy_bytes = (len(ids) - (cfg.n_local if args.merge == "stitched" else 0)) * eb
    remote_pulled = sum(1 for e in ids if e >= cfg.n_local) * eb
    gemm_gbps = alg_bytes / (gemm_ms * 1e-3) / 1e9
    gemm_tflops = alg_flop / (gemm_ms * 1e-3) / 1e12
    ai = alg_flop / alg_bytes
    if ai < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gemm_gbps / HBM_PEAK_GBPS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None}
    roof.update({"kernel": "moe_grouped_swiglu_combine (tile plan + gate/up GEMM + down GEMM with "
                           "the combine in its epilogue)" if comb else
                           "moe_grouped_swiglu (tile plan + gate/up GEMM + down GEMM)",
                 "avg_ms": round(gemm_ms, 4), "alg_bytes": alg_bytes, "alg_flop": alg_flop})
    tr = traffic_from_profiles(cfg.name)
    if tr is not None:
        roof["traffic"] = tr["hbm_bytes_per_call"]
        roof["traffic_detail"] = {"read": tr["read_bytes_per_call"], "write": tr["write_bytes_per_call"],
                                  "source": "profiles/grouped_swiglu_traffic.json"}

    result = {
        "metric": "MoE layer tokens/s + grouped-GEMM % of HBM/MFMA roofline, R1 shape, 1 GPU",
        "value": round(cfg.T * steps / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "local_experts": cfg.n_local,
                   "remote_fetch": args.remote, "copy_engine": args.copy_mode,
                   "copy_blocks": args.copy_blocks if args.copy_mode == "kernel" else None,
                   "merge": args.merge, "gather": args.gather, "combine": args.combine,
                   "fetch_chunks": nch, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "breakdown_ms": {"route_permute": round(rp_ms, 4), "merge_prefetch_copy": round(copy_ms, 4),
                         "grouped_swiglu": round(gemm_ms, 4), "combine": round(combine_ms, 4),
                         "layer_events": round(layer_ms, 4)},
        "timing": timing,
        "copy": {"bytes": copy_bytes, "experts": len(ids), "GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
                 "remote_pool": "pinned host" if remote_on_host else "device",
                 "remote_bytes": remote_pulled},
        "active_experts": n_active,
        "gemm_TFLOPs": round(gemm_tflops, 2),
        "hbm_frac": round(gemm_gbps / HBM_PEAK_GBPS, 4),
        "mfma_frac": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
    }
    if alt is not None:
        result["other_copy_engine"] = alt
    if graph_rec is not None:
        result["graph_replay"] = graph_rec
    if args.library_baseline and not remote_on_host:
        lb = library_baseline(L, cfg)
        lb["grouped_kernel_speedup"] = round(lb["ms"] / gemm_ms, 3)
        result["library_baseline"] = lb
    if cpu_sample > 0 and not comb:
        offs = L.offsets.cpu().numpy()
        src_of = L.src_of.cpu().numpy()
        active = np.nonzero(counts)[0]
        pick = np.sort(np.random.default_rng(cfg.seed + 7).choice(
            active, size=min(cpu_sample, len(active)), replace=False))
        x_h = synth.activations(cfg)
        rows = [np.arange(offs[e], offs[e + 1]) for e in pick]
        result["_cpu_sample"] = {
            "experts": [int(e) for e in pick], "n_active": int(len(active)), "R": int(R),
            "xp": np.concatenate([x_h[src_of[r] // cfg.k] for r in rows]),
            "off": np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64),
            "blocks": [block_to_numpy(L.expert_block(int(e))) for e in pick],
            "yp": np.concatenate([L.y_perm[int(offs[e]):int(offs[e + 1])].cpu().numpy()
                                  for e in pick])}
    if headline:
        result["inputs_sha256"] = input_digests(cfg, local, remote)
        result["_y"] = L.y.detach().cpu().numpy()
        if host_blocks is not None and not args.no_cpu_baseline:
            # host copies of the routed experts, taken outside every timed region
            for e in np.nonzero(counts)[0]:
                host_blocks[int(e)] = block_to_numpy(L.expert_block(int(e)))
    L.close()
    del L, local, remote
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    return result


if __name__ == "__main__":
    main()
