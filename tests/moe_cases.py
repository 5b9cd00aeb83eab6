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


def check_full(cfg, L, layer: int = 0, check_xperm: bool = True):
    """Whole-layer oracle on every token (small shapes); x_perm bitwise unless the layer
    gathers its rows on load (then x_perm is never written)."""
    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer)
    logits = synth.logits(cfg, layer)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(x, logits, cfg.k, weights_fn(L), cfg.H, cfg.I, round_h=cfg.dtype == "bf16")
    if check_xperm:
        assert out["x_perm"].tobytes() == np.asarray(ref["x_perm"]).tobytes()
    tol = TOL[cfg.dtype]
    e_yp = rel_err(out["y_perm"], ref["y_perm"])
    e_y = rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e} (tol {tol})")
    assert e_yp <= tol and e_y <= tol
    return out, ref


# ----------------------------------------------------------------------------
# full-size checks: many rows, each expert's weights read back and decoded once
# ----------------------------------------------------------------------------

def expert_ffn_rows(weights_of, x_rows_by_expert, H, I, round_h=True, workers=8):
    """The oracle's SwiGLU FFN of every expert e on its rows: {e: x rows} -> {e: float64 rows}.

    Each expert's block is fetched once (``weights_of`` on this thread) and decoded and
    multiplied on a worker thread, at most ``workers`` experts in flight (an R1 block decodes to
    352 MB of float64)."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    def work(bits, xr):
        wg, wu, wd = O.expert_matrices(bits, H, I)
        return O.swiglu_ffn(xr, wg, wu, wd, round_h)

    out, pending = {}, {}
    with threadpool_limits(limits=2), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for e in sorted(x_rows_by_expert):
            if len(pending) >= workers:
                done, _ = cf.wait(list(pending), return_when=cf.FIRST_COMPLETED)
                for f in done:
                    out[pending.pop(f)] = f.result()
            pending[ex.submit(work, weights_of(e), x_rows_by_expert[e])] = e
        for f in cf.as_completed(list(pending)):
            out[pending[f]] = f.result()
    return out


def tile_boundary_rows(offsets, step: int = 32):
    """Rows on both sides of every step-row boundary inside each expert's group, plus each
    group's first and last row.  Every tile of the grouped GEMM starts at a multiple of its
    32-row MFMA block from its expert's first row, so these include the first and last row of
    every tile, whatever tile heights the kernel picks."""
    rows = set()
    off = np.asarray(offsets, dtype=np.int64)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows.update((lo, hi - 1))
        for b in range(lo + step, hi, step):
            rows.update((b - 1, b))
    return sorted(rows)


def check_rows(cfg, L, rows, tokens, layer: int = 0, x=None, logits=None, check_xperm=True,
               workers=8):
    """Routing and permutation bit-exact on all tokens (and x_perm bitwise when built); y_perm
    on the given rows plus every row of the given tokens, and y on the given tokens, against
    the oracle's per-expert FFN of the rows (x read through the oracle's permutation).
    ``rows`` may be a function of the oracle's offsets (e.g. ``tile_boundary_rows``)."""
    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer) if x is None else x
    logits = synth.logits(cfg, layer) if logits is None else logits
    idx, w, src_of, row_of = check_routing(cfg, out, logits)
    if check_xperm:
        assert np.array_equal(out["x_perm"], np.asarray(x)[src_of // cfg.k])
    offsets = O.expert_offsets(O.expert_counts(idx, cfg.E))
    if callable(rows):
        rows = rows(offsets)
    tokens = [int(t) for t in tokens]
    tok_rows = [int(row_of[t * cfg.k + j]) for t in tokens for j in range(cfg.k)]
    rows = np.array(sorted(set(int(r) for r in rows) | set(tok_rows)), dtype=np.int64)
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    xa = np.asarray(x)
    by_e = {int(e): rows[e_of == e] for e in np.unique(e_of)}
    ffn = expert_ffn_rows(weights_fn(L), {e: xa[src_of[r] // cfg.k] for e, r in by_e.items()},
                          cfg.H, cfg.I, round_h=cfg.dtype == "bf16", workers=workers)
    ref = np.empty((len(rows), cfg.H))
    pos = {int(r): i for i, r in enumerate(rows)}
    for e, r in by_e.items():
        ref[[pos[int(v)] for v in r]] = ffn[e]
    tol = TOL[cfg.dtype]
    e_yp = rel_err(out["y_perm"][rows], ref)
    # y of the tokens: the oracle's combine over their k rows, in j order
    yp_tok = ref[[pos[r] for r in tok_rows]]
    y_ref = O.combine(yp_tok, np.arange(len(tok_rows)), w[tokens], cfg.k)
    e_y = rel_err(out["y"][tokens], y_ref)
    log(f"{cfg.name}: y_perm on {len(rows)} rows of {len(by_e)} experts: err/rms {e_yp:.3e}; "
        f"y on {len(tokens)} tokens: err/rms {e_y:.3e} (tol {tol})")
    assert e_yp <= tol and e_y <= tol
    return out, len(rows)


def check_every_row(cfg, L, layer: int = 0, x=None, logits=None, check_xperm=True, workers=8,
                    row_block: int = 8192):
    """Every row of y_perm and every token of y at any size: routing and permutation bit-exact
    on all tokens (x_perm bitwise when built); each active expert's rows through the oracle's
    float64 SwiGLU FFN (its block fetched once on this thread, decoded and multiplied on a
    worker thread, at most ``workers`` experts in flight, each writing its own rows of the
    float64 reference); y from the oracle's combine of those rows in j order.  The error is
    max|err| / RMS over all rows, taken ``row_block`` rows at a time so that no temporary of
    the full R x H size is made beside the reference."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer) if x is None else x
    logits = synth.logits(cfg, layer) if logits is None else logits
    idx, w, src_of, row_of = check_routing(cfg, out, logits)
    xa = np.asarray(x)
    if check_xperm:
        assert np.array_equal(out["x_perm"], xa[src_of // cfg.k])
    offsets = O.expert_offsets(O.expert_counts(idx, cfg.E))
    R = int(offsets[-1])
    ref = np.empty((R, cfg.H))
    round_h = cfg.dtype == "bf16"
    weights_of = weights_fn(L)

    def work(bits, lo, hi):
        wg, wu, wd = O.expert_matrices(bits, cfg.H, cfg.I)
        ref[lo:hi] = O.swiglu_ffn(xa[src_of[lo:hi] // cfg.k], wg, wu, wd, round_h)

    active = [e for e in range(cfg.E) if offsets[e + 1] > offsets[e]]
    pending = set()
    with threadpool_limits(limits=2), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for e in active:
            if len(pending) >= workers:
                done, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
                for f in done:
                    f.result()
            pending.add(ex.submit(work, weights_of(e), int(offsets[e]), int(offsets[e + 1])))
        for f in cf.as_completed(pending):
            f.result()
    yp = out["y_perm"]
    max_err, sumsq = 0.0, 0.0
    for r0 in range(0, R, row_block):
        g = yp[r0:r0 + row_block].astype(np.float64)
        rr = ref[r0:r0 + row_block]
        max_err = max(max_err, float(np.max(np.abs(g - rr))) if g.size else 0.0)
        sumsq += float(np.sum(rr * rr))
    e_yp = max_err / max(np.sqrt(sumsq / max(R * cfg.H, 1)), 1e-300)
    y_ref = O.combine(ref, row_of, w, cfg.k)
    e_y = rel_err(out["y"], y_ref)
    tol = TOL[cfg.dtype]
    log(f"{cfg.name}: y_perm on every one of {R} rows ({len(active)} experts): err/rms "
        f"{e_yp:.3e}; y on every one of {cfg.T} tokens: err/rms {e_y:.3e} (tol {tol})")
    assert e_yp <= tol and e_y <= tol
    return out, R


def tokens_layer(weights_of, x_rows, logits_rows, k, H, I, round_h=True, workers=8):
    """The oracle's layer output for a set of token rows: O.route of their logits, each chosen
    expert's FFN on its tokens (expert_ffn_rows: one decode per expert, experts in parallel),
    then O.combine over the k slots in j order.  The same value as O.moe_layer_tokens, which
    walks the experts one at a time."""
    xr = O.decode(x_rows)
    idx, w = O.route(logits_rows, k)
    n = xr.shape[0]
    flat = idx.ravel()
    by_e = {int(e): np.nonzero(flat == e)[0] for e in np.unique(flat)}
    ffn = expert_ffn_rows(weights_of, {e: xr[a // k] for e, a in by_e.items()}, H, I, round_h,
                          workers)
    yp = np.empty((n * k, H))
    for e, a in by_e.items():
        yp[a] = ffn[e]
    return O.combine(yp, np.arange(n * k), w, k)


def check_y_tokens(cfg, L, tokens, layer: int = 0, workers=8):
    """Routing and permutation bit-exact on all tokens; y of the given tokens against the
    oracle's per-token layer (for paths that write no y_perm)."""
    out = L.outputs()
    assert out["status"] == 0, f"device status {out['status']}"
    x = synth.activations(cfg, layer)
    logits = synth.logits(cfg, layer)
    check_routing(cfg, out, logits)
    tokens = [int(t) for t in tokens]
    y_ref = tokens_layer(weights_fn(L), np.asarray(x)[tokens], logits[tokens], cfg.k, cfg.H, cfg.I,
                         round_h=cfg.dtype == "bf16", workers=workers)
    e_y = rel_err(out["y"][tokens], y_ref)
    log(f"{cfg.name}: y on {len(tokens)} tokens: err/rms {e_y:.3e} (tol {TOL[cfg.dtype]})")
    assert e_y <= TOL[cfg.dtype]
    return out
