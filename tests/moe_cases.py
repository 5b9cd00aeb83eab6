"""Shared helpers of the GPU parity tests: build a layer on the GPU from the
seeded inputs, and compare its outputs with the CPU oracle.

Tolerances (written here, used by every GPU test):
* routing ids, counts, offsets, row_of, src_of, x_perm: bit-exact;
* routing weights: |w_gpu - w_oracle| <= 2e-6 (fp32 exp/divide vs float64);
* y and y_perm: max|err| <= 2e-2 * RMS(oracle) for bf16 weights with fp32
  accumulation, <= 1e-5 * RMS(oracle) for the fp32 workload.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import moe as O  # noqa: E402
from grouped_gemm_weights_amd import synth  # noqa: E402

W_TOL = 2e-6
TOL = {"bf16": 2e-2, "f32": 1e-5}


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def build_layer(cfg, layer: int = 0, host_weights: bool | None = None, remote_on_host: bool = False,
                **kw):
    """A MoELayer with seeded inputs and pools for ``cfg`` (weights drawn on the host for small
    shapes, on the device for R1 shapes)."""
    import torch
    from grouped_gemm_weights_amd.layer import MoELayer
    if host_weights is None:
        host_weights = cfg.H * cfg.I <= 1 << 20
    L = MoELayer(cfg, **kw)
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    if host_weights:
        def tpool(ids):
            a = synth.pool_np(cfg, layer, ids)
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            return t.view(tdt) if a.dtype == np.uint16 else t
        local = tpool(range(cfg.n_local)).cuda()
        remote = tpool(range(cfg.n_local, cfg.E))
        remote = remote.pin_memory() if remote_on_host else remote.cuda()
    else:
        local = synth.pool_torch(cfg, layer, 0, cfg.n_local, "cuda")
        remote = synth.pool_torch(cfg, layer, cfg.n_local, cfg.E - cfg.n_local, "cuda")
        if remote_on_host:
            remote = remote.cpu().pin_memory()
    L.set_pools(local, remote)
    L.set_inputs(synth.activations(cfg, layer), synth.logits(cfg, layer))
    return L


def weights_fn(L):
    from grouped_gemm_weights_amd.layer import block_to_numpy
    cache = {}

    def weights_of(e):
        if e not in cache:
            cache.clear()            # keep one decoded expert at a time (R1 blocks are 88 MB)
            cache[e] = block_to_numpy(L.expert_block(e))
        return cache[e]
    return weights_of


def rel_err(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / max(rms, 1e-300)


def bf16_ulp(v) -> np.ndarray:
    """Spacing of bf16 values at |v| (2**(e-8) for |v| in [2**(e-1), 2**e); 2**-133 below 2**-126)."""
    _, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def rel_err_bf16(got, ref, roundings: int = 1) -> float:
    """rel_err for outputs stored in bf16: both sides round to bf16 once at the end, so an
    element may differ by one bf16 spacing of the reference when the exact values fall on
    opposite sides of a rounding boundary; only the excess over that spacing counts.  A value
    re-rounded to bf16 at each of several stages may cross one boundary per stage
    (``roundings`` spacings)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    excess = np.maximum(np.abs(got - ref) - roundings * bf16_ulp(ref), 0.0)
    return float(np.max(excess)) / max(rms, 1e-300)


def check_routing(cfg, out, logits):
    """Bit-exact ids / counts / offsets / permutation and weights within W_TOL, on all tokens."""
    idx, w = O.route(logits, cfg.k)
    np.testing.assert_array_equal(out["idx"], idx)
    assert np.max(np.abs(out["w"].astype(np.float64) - w.astype(np.float64))) <= W_TOL
    counts = O.expert_counts(idx, cfg.E)
    np.testing.assert_array_equal(out["counts"], counts)
    np.testing.assert_array_equal(out["offsets"], O.expert_offsets(counts))
    row_of, src_of = O.permutation(idx, cfg.E)
    np.testing.assert_array_equal(out["src_of"], src_of)
    np.testing.assert_array_equal(out["row_of"], row_of)
    return idx, w, src_of, row_of


def check_full(cfg, L, layer: int = 0):
    """Whole-layer oracle on every token (small shapes)."""
    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer)
    logits = synth.logits(cfg, layer)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(x, logits, cfg.k, weights_fn(L), cfg.H, cfg.I, round_h=cfg.dtype == "bf16")
    assert out["x_perm"].tobytes() == np.asarray(ref["x_perm"]).tobytes()
    tol = TOL[cfg.dtype]
    e_yp = rel_err(out["y_perm"], ref["y_perm"])
    e_y = rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e} (tol {tol})")
    assert e_yp <= tol and e_y <= tol
    return out, ref


def check_sampled(cfg, L, tokens, layer: int = 0, x=None, logits=None, check_xperm=True):
    """Full routing/permutation parity, x_perm bitwise, y and y_perm on sampled tokens."""
    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer) if x is None else x
    logits = synth.logits(cfg, layer) if logits is None else logits
    idx, w, src_of, row_of = check_routing(cfg, out, logits)
    if check_xperm:
        assert np.array_equal(out["x_perm"], np.asarray(x)[src_of // cfg.k])
    ref = O.moe_layer_tokens(x, logits, cfg.k, weights_fn(L), cfg.H, cfg.I,
                             round_h=cfg.dtype == "bf16", tokens=tokens)
    tol = TOL[cfg.dtype]
    e_y = rel_err(out["y"][tokens], ref["y"])
    rows = np.array([row_of[t * cfg.k + j] for t in tokens for j in range(cfg.k)])
    yp_ref = ref["expert_out"].reshape(len(tokens) * cfg.k, cfg.H)
    e_yp = rel_err(out["y_perm"][rows], yp_ref)
    log(f"{cfg.name}: {len(tokens)} sampled tokens: y err/rms {e_y:.3e}, y_perm err/rms {e_yp:.3e}")
    assert e_y <= tol and e_yp <= tol
    return out
