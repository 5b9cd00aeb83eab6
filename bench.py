#!/usr/bin/env python3
"""Throughput of the DWDP-style MoE layer forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
with the weight pools and inputs already resident in HBM:

    route -> permute (counts, offsets, permutation, row gather)
    -> read the per-expert counts back (the routed remote set depends on them)
    -> copy stream: merge the local experts into the merged buffer half and
       prefetch the routed remote experts from the stand-in peer pool (SDMA)
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
    p.add_argument("--remote", choices=["routed", "all"], default="routed",
                   help="prefetch only the routed remote experts, or the whole remote share")
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
    p.add_argument("--merge", choices=["copy", "stitched"], default="stitched",
                   help="copy the local experts into each merged half, or stitch the local "
                        "block into the half's virtual range so the merge copies nothing")
    p.add_argument("--cpu-sample-tokens", type=int, default=24)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-single-thread-tokens", type=int, default=2,
                   help="tokens of the CPU sample also timed with the oracle held to one thread "
                        "(0: skip)")
    p.add_argument("--calibrate", action="store_true",
                   help="run only a plain streaming kernel of known size (moe_residual_add over "
                        "1 GiB elements), the reference for scaling the HBM byte counters")
    p.add_argument("--write-traffic", metavar="PROF_DIR",
                   help="no GPU work: turn rocprofv3 FETCH_SIZE / WRITE_SIZE csv runs under "
                        "PROF_DIR (fetch_<config>, write_<config>, cal_fetch, cal_write) for the "
                        "configs given with --traffic-configs into profiles/grouped_swiglu_traffic.json")
    p.add_argument("--traffic-configs", default="r1_decode_t64")
    return p.parse_args()


def cpu_baseline(cfg, L, n_tokens, single_thread_tokens=0):
    """The oracle as it stands, on a bounded sample: routing and permutation of all tokens,
    the layer output of n_tokens tokens (every expert they route to is decoded once)."""
    import numpy as np
    from oracle import moe as O
    from grouped_gemm_weights_amd import synth
    from grouped_gemm_weights_amd.layer import block_to_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = synth.activations(cfg)
    logits = synth.logits(cfg)
    tokens = list(range(min(n_tokens, cfg.T)))
    # expert blocks are host copies taken before the clock starts (the oracle reads host memory)
    idx, _ = O.route(logits[tokens], cfg.k)
    blocks = {int(e): block_to_numpy(L.expert_block(int(e))) for e in np.unique(idx)}
    t0 = time.perf_counter()
    idx_all, w_all = O.route(logits, cfg.k)
    counts = O.expert_counts(idx_all, cfg.E)
    O.expert_offsets(counts)
    O.permutation(idx_all, cfg.E)
    O.moe_layer_tokens(x, logits, cfg.k, lambda e: blocks[e], cfg.H, cfg.I,
                       round_h=cfg.dtype == "bf16", tokens=tokens)
    dt = time.perf_counter() - t0
    out = {"value": round(len(tokens) / dt, 4), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{len(tokens)} of {cfg.T} tokens through the float64 oracle "
                     f"(routing and permutation of all {cfg.T} tokens included), {dt:.1f} s",
           "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}
    if single_thread_tokens > 0:
        # the same oracle held to one BLAS thread, on a smaller sample of the same tokens
        from threadpoolctl import threadpool_limits
        few = tokens[:single_thread_tokens]
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            O.moe_layer_tokens(x, logits, cfg.k, lambda e: blocks[e], cfg.H, cfg.I,
                               round_h=cfg.dtype == "bf16", tokens=few)
            d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": round(len(few) / d1, 4), "unit": "tokens/s",
                                "sample": f"{len(few)} tokens, layer output only, {d1:.1f} s"}
    return out


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
                    fused_gather=args.gather == "fused")
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
            gemm.append(el(ev["wait1"][l], ev["g1"][l]))
            if l > 0:
                Lat.append(el(ev["m1"][l - 1], ev["m1"][l]))
    sev = mk()
    P.forward_serial(sev)
    torch.cuda.synchronize()
    C_alone = [el(sev["d0"][l], sev["m1"][l]) for l in range(n)]
    P.close()
    P_alone = [el(sev["c0"][l], sev["c1"][l]) for l in range(n)]
    mean = lambda v: float(np.mean(v))
    H = 1.0 - sum(stall) / sum(P_l)
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
    roof.update({"traffic": None, "kernel": "moe_grouped_swiglu, pipelined layers (with the copy running)",
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
                   "merge": args.merge, "gather": args.gather, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "pipeline": {
            "prefetch_ms": round(mean(P_l), 3), "prefetch_alone_ms": round(mean(P_alone), 3),
            "copy_bytes": (cfg.E - (cfg.n_local if P.stitched else 0)) * eb,
            "copy_GBps": round((cfg.E - (cfg.n_local if P.stitched else 0)) * eb / (mean(P_l) * 1e-3) / 1e9, 1),
            "stall_ms": round(mean(stall), 3), "hidden_fraction": round(H, 4),
            "compute_pipelined_ms": round(mean(comp_pipe), 3), "compute_alone_ms": round(mean(C_alone), 3),
            "contention_slowdown": round(mean(comp_pipe) / mean(C_alone), 3),
            "layer_latency_ms": round(mean(Lat), 3),
            "layer_latency_ms_median": round(float(np.median(Lat)), 3),
            "layer_latency_ms_min": round(float(np.min(Lat)), 3),
            "max_compute_prefetch_ms": round(max(mean(C_alone), mean(P_alone)), 3),
        },
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
                f"python3 bench.py --config {cfg} --steps 2 --warmup 1 --no-cpu-baseline",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write_{cfg} -o run -- "
                f"python3 bench.py --config {cfg} --steps 2 --warmup 1 --no-cpu-baseline",
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
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from grouped_gemm_weights_amd import binding as B
    from grouped_gemm_weights_amd import synth
    from grouped_gemm_weights_amd.layer import MoELayer

    cfg = synth.config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_mode = {"sdma": B.MOE_COPY_SDMA, "any": B.MOE_COPY_ANY,
                 "kernel": B.copy_kernel_on(args.copy_blocks)}[args.copy_mode]
    if cfg.layers != 1:
        print(json.dumps(bench_pipeline(args, cfg, dev, copy_mode)), flush=True)
        return
    L = MoELayer(cfg, device=dev, copy_mode=copy_mode, stitched=args.merge == "stitched",
                 fused_gather=args.gather == "fused")
    local = synth.pool_torch(cfg, 0, 0, cfg.n_local, dev)
    remote = synth.pool_torch(cfg, 0, cfg.n_local, cfg.E - cfg.n_local, dev)
    L.set_pools(local, remote)
    L.set_inputs(synth.activations(cfg), synth.logits(cfg))
    cs, ps = L.compute_stream, L.copy_stream

    nev = args.steps
    mk = lambda: [B.moe_event_create(True) for _ in range(nev)]
    ev = {k: mk() for k in ("start", "rp_end", "gemm0", "gemm1", "end", "copy0", "copy1")}
    nch = max(0, args.chunks)
    gev = [{"g0": [B.moe_event_create(True) for _ in range(nch + 1)],
            "g1": [B.moe_event_create(True) for _ in range(nch + 1)]} for _ in range(nev)]

    def step(i, timed):
        h = i % 2
        if timed:
            B.moe_event_record(ev["start"][i], cs)
        L.route_permute()
        if timed:
            B.moe_event_record(ev["rp_end"][i], cs)
        ids = L.routed_ids() if args.remote == "routed" else list(range(cfg.E))
        if timed:
            B.moe_event_record(ev["copy0"][i], ps)
        if nch > 0:
            L.forward_chunked(h, ids, nch, gev[i] if timed else None)
            if timed:
                B.moe_event_record(ev["copy1"][i], ps)
                B.moe_event_record(ev["end"][i], cs)
            return ids
        L.fill_half(h, ids)
        if timed:
            B.moe_event_record(ev["copy1"][i], ps)
        B.moe_stream_wait_event(cs, L.ready[h])
        if timed:
            B.moe_event_record(ev["gemm0"][i], cs)
        L.grouped(L.wbufs[h])
        if timed:
            B.moe_event_record(ev["gemm1"][i], cs)
        B.moe_combine(L.y_perm, L.row_of, L.topk_w, cfg.T, cfg.k, cfg.H, L.y, cs)
        B.moe_event_record(L.free[h], cs)
        if timed:
            B.moe_event_record(ev["end"][i], cs)
        return ids

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ids = step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert L.read_status() == 0, "device status set during the benchmark"
    alt = None
    if args.alt_steps > 0:
        # the same step with the other copy path, for comparison (not the reported value)
        alt_name = "sdma" if args.copy_mode == "any" else "any"
        L.copy_mode = B.MOE_COPY_SDMA if alt_name == "sdma" else B.MOE_COPY_ANY
        for i in range(2):
            step(i, False)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for i in range(args.alt_steps):
            step(i, False)
        torch.cuda.synchronize()
        alt_s = (time.perf_counter() - ta) / args.alt_steps
        alt = {"copy_engine": alt_name,
               "ms_per_step": round(alt_s * 1e3, 3), "tokens_per_s": round(cfg.T / alt_s, 1)}
        L.copy_mode = copy_mode

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

    counts = L.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    eb = synth.expert_block_bytes(cfg)
    R = cfg.T * cfg.k
    alg_bytes = n_active * eb + R * cfg.H * 2 + R * cfg.H * 4       # weights read + x_perm + y_perm
    alg_flop = 6.0 * cfg.H * cfg.I * R
    copy_bytes = (len(ids) - (cfg.n_local if args.merge == "stitched" else 0)) * eb
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
    roof.update({"kernel": "moe_grouped_swiglu (tile plan + gate/up GEMM + down GEMM)",
                 "avg_ms": round(gemm_ms, 4), "alg_bytes": alg_bytes, "alg_flop": alg_flop})
    tr = traffic_from_profiles(cfg.name)
    if tr is not None:
        roof["traffic"] = tr["hbm_bytes_per_call"]
        roof["traffic_detail"] = {"read": tr["read_bytes_per_call"], "write": tr["write_bytes_per_call"],
                                  "source": "profiles/grouped_swiglu_traffic.json"}

    result = {
        "metric": "MoE layer tokens/s + grouped-GEMM % of HBM/MFMA roofline, R1 shape, 1 GPU",
        "value": round(cfg.T * args.steps / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "local_experts": cfg.n_local,
                   "remote_fetch": args.remote, "copy_engine": args.copy_mode,
                   "copy_blocks": args.copy_blocks if args.copy_mode == "kernel" else None,
                   "merge": args.merge, "gather": args.gather, "fetch_chunks": nch, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "breakdown_ms": {"route_permute": round(rp_ms, 4), "merge_prefetch_copy": round(copy_ms, 4),
                         "grouped_swiglu": round(gemm_ms, 4), "combine": round(combine_ms, 4),
                         "layer_events": round(layer_ms, 4)},
        "timing": timing,
        "copy": {"bytes": copy_bytes, "experts": len(ids), "GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1)},
        "active_experts": n_active,
        "gemm_TFLOPs": round(gemm_tflops, 2),
    }
    if alt is not None:
        result["other_copy_engine"] = alt
    result["inputs_sha256"] = input_digests(cfg, local, remote)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, L, args.cpu_sample_tokens,
                                              args.cpu_single_thread_tokens)
    L.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
