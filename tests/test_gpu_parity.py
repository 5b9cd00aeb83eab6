"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every test runs the library on seeded inputs and compares with the oracle
element by element: bit-exact for routing ids, counts, offsets, the
permutation and the gathered rows; within the tolerances of tests/moe_cases.py
for the routing weights and the float outputs.  Shapes span several tiles
with ragged tails.  The DeepSeek-R1-shaped workloads run at full size and are
checked on every row of y_perm and every token of y.
"""
import gc

import numpy as np
import pytest

from moe_cases import (O, TOL, build_layer, check_every_row, check_full, check_routing,
                       check_rows, check_y_tokens, log, rel_err, synth, weights_fn)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _run(L, remote="routed"):
    L.forward(half=0, remote=remote)
    return L


# ----------------------------------------------------------------------------
# small shapes: whole-layer oracle on every token
# ----------------------------------------------------------------------------

def test_tiny_fp32_layer():
    cfg = synth.config("tiny_fp32_t64")
    log(f"case {cfg}")
    L = _run(build_layer(cfg))
    check_full(cfg, L)


@pytest.mark.parametrize("T,H,I,E,k,n_local,zipf", [
    (50, 136, 72, 37, 3, 9, None),        # nothing a multiple of the tile sizes
    (33, 264, 200, 16, 4, 4, 1.1),       # skewed routing, zero-count experts
    (300, 128, 64, 8, 2, 2, None),        # many rows per expert: prefill tiles, ragged tail
    (1, 64, 32, 5, 2, 1, None),           # a single token
    (64, 256, 512, 8, 1, 4, None),        # k = 1
    (40, 96, 40, 70, 8, 20, 1.1),         # E above one wave, skew
    (16, 136, 72, 37, 3, 9, None),        # decode tiles: K and N tails (K % 128, N % 32 != 0)
    (24, 256, 512, 64, 8, 16, None),      # decode tiles, full 128-deep K steps
    (12, 1024, 200, 40, 6, 10, 1.1),      # decode tiles, skew, K = 1024
])
def test_small_bf16_layers(T, H, I, E, k, n_local, zipf):
    cfg = synth.MoEConfig(f"bf16_T{T}_H{H}_I{I}_E{E}_k{k}", T=T, H=H, I=I, E=E, k=k, dtype="bf16",
                          n_local=n_local, seed=1000 + T + E, zipf_s=zipf, rho_seed=7)
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg))
    out, ref = check_full(cfg, L)
    if k == 1:
        # weight 1.0: the combine is an exact copy of the expert row
        np.testing.assert_array_equal(out["y"], out["y_perm"][out["row_of"]])


@pytest.mark.parametrize("T,H,I,E,k,n_local,stitched", [
    (20, 64, 32, 4, 4, 2, False),          # k = E: every token picks every expert
    (30, 64, 32, 1, 1, 1, False),          # a single expert, all local
    (16, 64, 32, 1024, 8, 256, False),     # E at the kernel limit (MOE_MAX_E)
    (8, 64, 32, 64, 64, 16, False),        # k at the kernel limit (MOE_MAX_K)
    (40, 64, 32, 16, 2, 0, False),         # every expert remote (empty local pool)
    (40, 64, 32, 16, 2, 16, False),        # every expert local (empty remote pool)
    (24, 1024, 1024, 8, 2, 0, True),       # stitched half with no local block
    (24, 1024, 1024, 8, 2, 8, True),       # stitched half with no fetched block
], ids=["k_eq_E", "one_expert", "E_max", "k_max", "all_remote", "all_local",
        "stitched_all_remote", "stitched_all_local"])
def test_edge_layers(T, H, I, E, k, n_local, stitched):
    cfg = synth.MoEConfig(f"bf16_edge_T{T}_E{E}_k{k}_l{n_local}", T=T, H=H, I=I, E=E, k=k,
                          dtype="bf16", n_local=n_local, seed=77 + T + E)
    log(f"case {cfg.name} stitched={stitched}")
    L = build_layer(cfg, stitched=stitched)
    try:
        _run(L)
        out, ref = check_full(cfg, L)
        assert out["counts"].sum() == T * k
        if k == E:
            np.testing.assert_array_equal(out["counts"], np.full(E, T))
    finally:
        L.close()


def test_empty_batch():
    cfg = synth.MoEConfig("bf16_empty", T=0, H=64, I=32, E=8, k=2, dtype="bf16", n_local=4, seed=5)
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg))
    out = L.outputs()
    assert out["status"] == 0
    np.testing.assert_array_equal(out["counts"], np.zeros(cfg.E, np.int32))
    np.testing.assert_array_equal(out["offsets"], np.zeros(cfg.E + 1, np.int32))
    assert out["y"].shape == (0, cfg.H) and out["y_perm"].shape == (0, cfg.H)


def test_all_tokens_one_expert_and_prefill_tiles():
    cfg = synth.MoEConfig("bf16_one_hot", T=700, H=128, I=96, E=12, k=2, dtype="bf16", n_local=3,
                          seed=5)
    log(f"case {cfg.name}")
    L = build_layer(cfg)
    logits = synth.logits(cfg)
    logits[:, 7] += 50.0                   # every token picks expert 7 first
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=1)
    out = L.outputs()
    assert out["counts"][7] == cfg.T
    idx, w, src_of, row_of = check_routing(cfg, out, logits)
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    assert rel_err(out["y"], ref["y"]) <= TOL["bf16"]


def _random_cases(n, seed):
    """Seeded layer shapes: T, H, I, E, k, the local split, skew, gather and pull modes."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 16, 37, 64, 100, 256, 300]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([1, 3, 17, 64, 130, 333, 600]))
        H = 8 * int(rng.integers(1, 65))
        I = 8 * int(rng.integers(1, 49))
        cases.append(dict(T=T, H=H, I=I, E=E, k=k, n_local=int(rng.integers(0, E + 1)),
                          zipf=float(rng.choice([0.0, 1.1])), fused=bool(rng.integers(0, 2)),
                          remote=str(rng.choice(["routed", "device", "all"])), seed=int(seed * 100 + i)))
    return cases


def test_random_layer_shapes():
    """Forty seeded layer shapes, each checked against the whole-layer oracle on every token:
    H and I any multiples of 8 up to 512 and 384, E from 1 to 300, k up to 16, T from 1 to
    600, any local split, uniform or Zipf-skewed routing, x_perm or the fused gather, and the
    three pull modes."""
    for c in _random_cases(40, 61):
        cfg = synth.MoEConfig(f"bf16_rand{c['seed']}", T=c["T"], H=c["H"], I=c["I"], E=c["E"],
                              k=c["k"], dtype="bf16", n_local=c["n_local"], seed=c["seed"],
                              zipf_s=c["zipf"] or None)
        log(f"case {cfg.name}: T={c['T']} H={c['H']} I={c['I']} E={c['E']} k={c['k']} "
            f"n_local={c['n_local']} zipf={c['zipf']} fused={c['fused']} remote={c['remote']}")
        L = build_layer(cfg, fused_gather=c["fused"])
        try:
            L.forward(half=0, remote=c["remote"])
            L.synchronize()
            check_full(cfg, L, check_xperm=not c["fused"])
        finally:
            L.close()
        del L
        gc.collect()


def test_random_fp32_layer_shapes():
    """Sixteen seeded fp32 layers of any H and I (1 to 300, so expert blocks of any byte size),
    each checked against the whole-layer oracle on every token at the fp32 tolerance; the
    device-routed pull where the blocks are whole 16-byte words, else the host-routed one."""
    rng = np.random.default_rng(62)
    for i in range(16):
        E = int(rng.choice([1, 3, 8, 33, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T, H, I = int(rng.choice([1, 5, 40, 129])), int(rng.integers(1, 301)), int(rng.integers(1, 301))
        remote = "device" if (3 * H * I * 4) % 16 == 0 else str(rng.choice(["routed", "all"]))
        cfg = synth.MoEConfig(f"f32_rand{6200 + i}", T=T, H=H, I=I, E=E, k=k, dtype="f32",
                              n_local=int(rng.integers(0, E + 1)), seed=6200 + i,
                              zipf_s=float(rng.choice([0.0, 1.1])) or None)
        fused = bool(rng.integers(0, 2))
        log(f"case {cfg.name}: T={T} H={H} I={I} E={E} k={k} n_local={cfg.n_local} "
            f"fused={fused} remote={remote}")
        L = build_layer(cfg, fused_gather=fused)
        try:
            L.forward(half=0, remote=remote)
            L.synchronize()
            check_full(cfg, L, check_xperm=not fused)
        finally:
            L.close()
        del L
        gc.collect()


def _tied_logits(cfg, seed):
    """Logits with ties everywhere: N(0,1) rounded to multiples of 0.5, plus rows of one repeated
    value, rows of +0.0 and -0.0 mixed (equal under the routing order), rows where a run of
    equal values straddles the k-th place, and a row of -0.0 with one +0.0 at the end."""
    rng = np.random.default_rng(seed)
    L = (np.round(rng.standard_normal((cfg.T, cfg.E)) * 2.0) / 2.0).astype(np.float32)
    T, E, k = cfg.T, cfg.E, cfg.k
    L[0, :] = 1.5                                              # all equal: ids 0..k-1, w = 1/k
    L[1, :] = np.where(rng.random(E) < 0.5, 0.0, -0.0).astype(np.float32)
    L[2, :] = -0.0
    L[2, E - 1] = 0.0                                          # +0 == -0: still ids 0..k-1
    L[3, :] = -1.0
    L[3, E // 2:] = 2.0                                        # equal top values from the middle
    L[4, :] = 0.5
    L[4, rng.choice(E, size=max(1, k // 2), replace=False)] = 3.0   # a run straddling place k
    for t in range(5, min(T, 12)):                             # signed zeros in quantised rows
        z = rng.choice(E, size=E // 3, replace=False)
        L[t, z] = np.where(rng.random(z.size) < 0.5, 0.0, -0.0)
    return L


@pytest.mark.parametrize("E,k,H,I", [(256, 8, 64, 32), (8, 2, 64, 32), (1000, 8, 64, 32)],
                         ids=["E256_k8", "E8_k2", "E1000_k8"])
def test_routing_ties_and_signed_zeros(E, k, H, I):
    """Quantised logits tie constantly; the order (logit desc, id asc, +0 == -0) must pick the
    oracle's ids bit-exactly, and counts, offsets and the permutation with them.  The whole
    layer is checked too."""
    cfg = synth.MoEConfig(f"bf16_ties_E{E}_k{k}", T=200, H=H, I=I, E=E, k=k, dtype="bf16",
                          n_local=E // 4, seed=31 + E)
    log(f"case {cfg.name}")
    L = build_layer(cfg)
    logits = _tied_logits(cfg, 32 + E)
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=0)
    out = L.outputs()
    assert out["status"] == 0
    idx, w, src_of, row_of = check_routing(cfg, out, logits)
    np.testing.assert_array_equal(out["idx"][0], np.arange(k))
    np.testing.assert_array_equal(out["idx"][2], np.arange(k))
    assert np.max(np.abs(out["w"][0] - 1.0 / k)) <= 2e-7
    ties = sum(int(np.sum(logits[t] == logits[t, idx[t, -1]]) > 1) for t in range(cfg.T))
    log(f"{cfg.name}: {ties} of {cfg.T} tokens have a tie at the k-th place")
    assert ties > cfg.T // 4
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    e_y = rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y err/rms {e_y:.3e}")
    assert e_y <= TOL["bf16"]


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_prefill_tile_modes_at_row_boundaries(fused):
    """Expert row counts on both sides of every prefill tile mode (32/64/128/192-row
    column-split tiles, full 256-row tiles, and a full tile plus a one-row tail), k = 1 so each
    count is exact; I = 192 leaves the gate/up GEMM a partial column block, so the epilogue
    runs both its unchecked (whole waves) and checked stores."""
    counts = [1, 32, 33, 64, 65, 128, 129, 192, 193, 256, 257]
    T = sum(counts)
    cfg = synth.MoEConfig("bf16_tile_modes", T=T, H=256, I=192, E=len(counts), k=1, dtype="bf16",
                          n_local=3, seed=21)
    log(f"case {cfg.name} fused={fused}")
    L = build_layer(cfg, fused_gather=fused)
    expert_of = np.repeat(np.arange(cfg.E), counts)
    np.random.default_rng(22).shuffle(expert_of)       # tokens of an expert spread over the batch
    logits = synth.logits(cfg)
    logits[np.arange(T), expert_of] += 50.0
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=0)
    out = L.outputs()
    assert out["status"] == 0
    np.testing.assert_array_equal(out["counts"], counts)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    e_yp, e_y = rel_err(out["y_perm"], ref["y_perm"]), rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e}")
    assert e_yp <= TOL["bf16"] and e_y <= TOL["bf16"]


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_prefill_multi_tile_experts(fused):
    """Experts of 511, 512, 513, 1024 and 1025 rows (k = 1): a full 256-row tile and a 255-row
    one, exactly two, two plus a one-row tail (a 64-row column-split tile), four, four plus one
    row; H = 256 and I = 192 as above.  Every row is checked."""
    counts = [511, 512, 513, 1024, 1025, 3, 0]
    T = sum(counts)
    cfg = synth.MoEConfig("bf16_multi_tile", T=T, H=256, I=192, E=len(counts), k=1, dtype="bf16",
                          n_local=2, seed=29)
    log(f"case {cfg.name} fused={fused}")
    L = build_layer(cfg, fused_gather=fused)
    expert_of = np.repeat(np.arange(cfg.E), counts)
    np.random.default_rng(30).shuffle(expert_of)
    logits = synth.logits(cfg)
    logits[np.arange(T), expert_of] += 50.0
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=0)
    out = L.outputs()
    assert out["status"] == 0
    np.testing.assert_array_equal(out["counts"], counts)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    e_yp, e_y = rel_err(out["y_perm"], ref["y_perm"]), rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e}")
    assert e_yp <= TOL["bf16"] and e_y <= TOL["bf16"]


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_prefill_hot_expert_runs(fused):
    """Hot experts whose heavy tiles fill runs of aligned heavy groups, which the prefill GEMM
    regroups into more m-tiles by fewer n-tiles each: 8 full tiles plus a tail (a run of four
    groups), 4 plus a tail and 4 (runs of two), 2 plus a tail (no run), with I = 512 and
    H = 1024 so that both GEMMs have 4 n-tiles and both run lengths apply (k = 1).  Every row
    is checked."""
    counts = [2100, 1100, 1024, 700, 3, 0]
    T = sum(counts)
    cfg = synth.MoEConfig("bf16_hot_runs", T=T, H=1024, I=512, E=len(counts), k=1, dtype="bf16",
                          n_local=2, seed=31)
    log(f"case {cfg.name} fused={fused}")
    L = build_layer(cfg, fused_gather=fused)
    expert_of = np.repeat(np.arange(cfg.E), counts)
    np.random.default_rng(32).shuffle(expert_of)
    logits = synth.logits(cfg)
    logits[np.arange(T), expert_of] += 50.0
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=0)
    out = L.outputs()
    assert out["status"] == 0
    np.testing.assert_array_equal(out["counts"], counts)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    e_yp, e_y = rel_err(out["y_perm"], ref["y_perm"]), rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e}")
    assert e_yp <= TOL["bf16"] and e_y <= TOL["bf16"]


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_decode_tiles_at_row_boundaries(fused):
    """Decode-path layer (at most 4 rows per expert on average) with expert row counts around
    the 16-row stream tile (1, 15, 16, 17, 32, 33), k = 1; H = 320 and I = 192 give both stream
    GEMMs a partial column block and a K tail (neither depth is a multiple of 128)."""
    counts = [1, 15, 16, 17, 32, 33] + [0] * 26
    T = sum(counts)
    cfg = synth.MoEConfig("bf16_decode_tiles", T=T, H=320, I=192, E=len(counts), k=1,
                          dtype="bf16", n_local=8, seed=23)
    assert T <= 4 * cfg.E                      # the decode tiles are chosen
    log(f"case {cfg.name} fused={fused}")
    L = build_layer(cfg, fused_gather=fused)
    expert_of = np.repeat(np.arange(cfg.E), counts)
    np.random.default_rng(24).shuffle(expert_of)
    logits = synth.logits(cfg)
    logits[np.arange(T), expert_of] += 50.0
    L.set_inputs(synth.activations(cfg), logits)
    L.forward(half=1)
    out = L.outputs()
    assert out["status"] == 0
    np.testing.assert_array_equal(out["counts"], counts)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(synth.activations(cfg), logits, cfg.k, weights_fn(L), cfg.H, cfg.I, True)
    e_yp, e_y = rel_err(out["y_perm"], ref["y_perm"]), rel_err(out["y"], ref["y"])
    log(f"{cfg.name}: y_perm err/rms {e_yp:.3e}, y err/rms {e_y:.3e}")
    assert e_yp <= TOL["bf16"] and e_y <= TOL["bf16"]


def test_late_prefetch_is_waited_for():
    """The compute stream waits for the copy stream's ready event: with the half poisoned with
    NaN and the copy stream held back by a spin kernel queued before the pull, the layer's
    output is bit-identical to an undelayed run and the step's time grows by about the
    delay (a missing or misplaced wait would read NaN weights)."""
    cfg = synth.MoEConfig("bf16_late_prefetch", T=256, H=512, I=256, E=16, k=4, dtype="bf16",
                          n_local=4, seed=25)
    log(f"case {cfg.name}")
    L = build_layer(cfg)
    cs, ps = L.compute_stream, L.copy_stream
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed_step(delay_cycles):
        base, _ = L.halves[0]
        base.fill_(0xFF)                               # bf16 0xFFFF is NaN
        torch.cuda.synchronize()
        d0, d1, c0, c1 = ev(), ev(), ev(), ev()
        d0.record(ps)
        if delay_cycles:
            with torch.cuda.stream(ps):
                torch.cuda._sleep(delay_cycles)
        d1.record(ps)
        c0.record(cs)
        L.forward(half=0)
        c1.record(cs)
        torch.cuda.synchronize()
        return L.outputs(), d0.elapsed_time(d1), c0.elapsed_time(c1)

    timed_step(0)                                      # warm-up
    ref, _, t_base = timed_step(0)
    assert ref["status"] == 0 and np.isfinite(ref["y"]).all()
    late, delay, t_late = timed_step(20_000_000)
    log(f"delay {delay:.2f} ms: step {t_base:.2f} -> {t_late:.2f} ms")
    assert late["status"] == 0
    assert late["y"].tobytes() == ref["y"].tobytes()
    assert delay >= 2.0
    assert t_late - t_base >= 0.5 * delay


@pytest.mark.parametrize("remote", ["routed", "device"])
def test_injected_prefetch_fault_surfaces_and_recovers(monkeypatch, remote):
    """MOE_INJECT_FAULT=prefetch: the layer step raises the library's error instead of running
    the GEMM on a half that was never filled (host-routed pull, or the device-routed one);
    without it the next step is correct."""
    from grouped_gemm_weights_amd import binding as B
    cfg = synth.MoEConfig("bf16_fault", T=64, H=128, I=64, E=12, k=3, dtype="bf16", n_local=3,
                          seed=27)
    log(f"case {cfg.name} remote={remote}")
    L = build_layer(cfg)
    monkeypatch.setenv("MOE_INJECT_FAULT", "prefetch")
    with pytest.raises(B.MoEError) as e:
        L.forward(half=0, remote=remote)
    assert e.value.code == B.MOE_ERR_HIP
    assert ("moe_prefetch_routed" if remote == "device" else "moe_prefetch_layer") in str(e.value)
    monkeypatch.delenv("MOE_INJECT_FAULT")
    L.synchronize()
    L.forward(half=0, remote=remote)
    check_full(cfg, L)


def test_remote_pool_in_pinned_host_memory():
    cfg = synth.MoEConfig("bf16_host_remote", T=48, H=128, I=64, E=16, k=4, dtype="bf16",
                          n_local=4, seed=9)
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg, remote_on_host=True))
    check_full(cfg, L)


def _check_device_slot_map(cfg, L, half, check_bytes=False):
    """slot_of after a device-routed fill: e for local experts and routed remote ones, -1 else;
    with check_bytes, the slot of every local and routed remote expert holds exactly that
    expert's block of its pool."""
    counts = L.counts.cpu().numpy()
    want = np.array([e if (e < cfg.n_local or counts[e] > 0) else -1 for e in range(cfg.E)],
                    dtype=np.int32)
    np.testing.assert_array_equal(L.slot_maps[half].cpu().numpy(), want)
    if check_bytes:
        base = L.halves[half][0]
        if isinstance(base, int):          # a stitched half: a raw device range, viewed by torch

            class _Range:
                __cuda_array_interface__ = {"shape": (L.n_slots * L.eb,), "typestr": "|u1",
                                            "data": (base, False), "version": 3}
            base = torch.as_tensor(_Range(), device="cuda")
        got = base.view(torch.uint8).reshape(L.n_slots, L.eb).cpu().numpy()
        for e in np.nonzero(want >= 0)[0]:
            blk = L.expert_block(int(e)).contiguous().view(torch.uint8).cpu().numpy().reshape(-1)
            assert got[e].tobytes() == blk.tobytes(), f"slot {e}"


@pytest.mark.parametrize("T,H,I,E,k,n_local,zipf,stitched", [
    (40, 128, 64, 16, 2, 4, None, False),    # prefill-like tiles
    (40, 128, 64, 16, 2, 4, None, True),
    (12, 1024, 200, 40, 6, 10, 1.1, False),  # decode tiles, skew: many remote experts get no token
    (12, 1024, 200, 40, 6, 10, 1.1, True),
    (24, 64, 32, 16, 2, 0, None, False),     # no local experts
    (24, 64, 32, 16, 2, 16, None, False),    # no remote experts
], ids=["prefill-copy", "prefill-stitched", "decode-skew-copy", "decode-skew-stitched",
        "no-local", "no-remote"])
def test_device_routed_pull(T, H, I, E, k, n_local, zipf, stitched):
    """The routed pull decided on the device (moe_prefetch_routed): the slot map, the layer
    against the oracle, and y bit-equal to the host-routed pull's on the other half; then a
    second step with other logits on the same half."""
    cfg = synth.MoEConfig(f"bf16_devroute_T{T}_E{E}_l{n_local}", T=T, H=H, I=I, E=E, k=k,
                          dtype="bf16", n_local=n_local, seed=400 + T + E, zipf_s=zipf)
    log(f"case {cfg.name} stitched={stitched}")
    L = build_layer(cfg, stitched=stitched)
    try:
        L.forward(half=0, remote="device")
        L.synchronize()
        _check_device_slot_map(cfg, L, 0, check_bytes=True)
        check_full(cfg, L)
        y_dev = L.y.clone()
        torch.cuda.synchronize()
        L.forward(half=1, remote="routed")
        L.synchronize()
        assert torch.equal(L.y, y_dev)
        # other logits, same half: entries of experts routed only in the first step go back to -1
        L.set_inputs(synth.activations(cfg, 1), synth.logits(cfg, 1))
        L.forward(half=0, remote="device")
        L.synchronize()
        _check_device_slot_map(cfg, L, 0, check_bytes=True)
        check_full(cfg, L, layer=1)
    finally:
        L.close()


@pytest.mark.parametrize("stitched", [False, True], ids=["copy-merge", "stitched-merge"])
def test_device_routed_step_graph_replay(stitched):
    """The whole device-routed step captured into a HIP graph: four replays, with eager work
    and synchronisations between them, each bit-equal to the eager step; then new inputs
    written in place and one more replay checked against the oracle."""
    cfg = synth.MoEConfig("bf16_graph_step", T=24, H=1024, I=256, E=32, k=4, dtype="bf16",
                          n_local=8, seed=77, zipf_s=1.1)
    log(f"case {cfg.name} stitched={stitched}")
    L = build_layer(cfg, stitched=stitched, fused_gather=True)
    try:
        L.forward(half=0, remote="device")
        L.synchronize()
        check_full(cfg, L, check_xperm=False)
        y0 = L.y.clone()
        g = L.capture_step(half=0)
        for r in range(4):
            L.y.fill_(float("nan"))           # eager work between replays
            L.y_perm.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(L.y, y0), f"replay {r}"
        L.set_inputs(synth.activations(cfg, 1), synth.logits(cfg, 1))
        g.replay()
        torch.cuda.synchronize()
        _check_device_slot_map(cfg, L, 0, check_bytes=True)
        check_full(cfg, L, layer=1, check_xperm=False)
        del g
    finally:
        L.close()


def test_merged_buffer_bytes_and_slot_map():
    cfg = synth.MoEConfig("bf16_merge", T=40, H=64, I=32, E=20, k=3, dtype="bf16", n_local=5, seed=3)
    L = build_layer(cfg)
    ids = [0, 1, 3, 4, 6, 7, 8, 19]
    base, slot_of = L.halves[1]
    base.fill_(0xFF)                       # poison: bf16 0xFFFF is NaN
    torch.cuda.synchronize()
    L.fill_half(1, ids, wait_free=False)
    L.synchronize()
    np.testing.assert_array_equal(slot_of.cpu().numpy(), O.slot_map(ids, cfg.E))
    pools = [(0, L._local_t.cpu().view(torch.int16).numpy()),
             (cfg.n_local, L._remote_t.cpu().view(torch.int16).numpy())]
    merged = O.merge(pools, ids)
    got = base.cpu().numpy()[: len(ids)].view(np.int16)
    assert got.tobytes() == merged.tobytes()
    # the runtime's copy and the library's copy kernel (one workgroup, and unbounded)
    # give the same bytes
    from grouped_gemm_weights_amd import binding as B
    for mode in (B.MOE_COPY_ANY, B.MOE_COPY_SDMA, B.copy_kernel_on(1), B.copy_kernel_on(0)):
        base.fill_(0)
        torch.cuda.synchronize()
        B.moe_merge_weights(L.local_pool, ids, L.wbufs[1], L.copy_stream, copy_mode=mode)
        B.moe_prefetch_layer(L.remote_pool, ids, L.wbufs[1], L.copy_stream, copy_mode=mode)
        L.synchronize()
        assert base.cpu().numpy()[: len(ids)].view(np.int16).tobytes() == merged.tobytes(), mode


@pytest.mark.parametrize("mode", ["kernel", "any"])
def test_fp32_odd_blocks_every_copy_path(mode):
    """fp32 expert blocks of 3*5*3*4 = 180 bytes: not a multiple of 16, so the copy kernel
    hands each run to the runtime copy; the layer still matches the oracle."""
    from grouped_gemm_weights_amd import binding as B
    cfg = synth.MoEConfig("f32_odd_blocks", T=24, H=5, I=3, E=6, k=2, dtype="f32", n_local=2,
                          seed=21)
    log(f"case {cfg.name} copy={mode}")
    L = build_layer(cfg, copy_mode=B.MOE_COPY_KERNEL if mode == "kernel" else B.MOE_COPY_ANY)
    _run(L)
    check_full(cfg, L)


# ----------------------------------------------------------------------------
# error paths reported through the device status word
# ----------------------------------------------------------------------------

def test_status_nonfinite_logit_and_absent_expert():
    from grouped_gemm_weights_amd import binding as B
    cfg = synth.MoEConfig("bf16_status", T=16, H=64, I=32, E=8, k=2, dtype="bf16", n_local=2, seed=4)
    L = build_layer(cfg)
    logits = synth.logits(cfg)
    logits[3, 5] = np.nan
    L.set_inputs(synth.activations(cfg), logits)
    L.route_permute()
    assert L.read_status() & B.MOE_STATUS_NONFINITE_LOGIT
    # valid logits, but a routed remote expert left out of the merged buffer
    L.status.zero_()                       # set_inputs synchronises torch's stream
    L.set_inputs(synth.activations(cfg), synth.logits(cfg))
    L.route_permute()
    ids = L.routed_ids()
    missing = ids[-1]
    L.fill_half(0, [e for e in ids if e != missing])
    L.expert_compute(0)
    st = L.read_status()
    assert st & B.MOE_STATUS_EXPERT_ABSENT and not st & B.MOE_STATUS_NONFINITE_LOGIT
    # a slot map entry past the merged buffer is reported as absent and never read
    L.status.zero_()
    L.fill_half(0, ids)
    L.synchronize()
    _, slot_of = L.halves[0]
    slot_of[missing] = L.n_slots + 5
    torch.cuda.synchronize()
    L.expert_compute(0)
    st = L.read_status()
    assert st == B.MOE_STATUS_EXPERT_ABSENT


# ----------------------------------------------------------------------------
# DeepSeek-R1-shaped workloads at full size
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("stitched", [False, True], ids=["copy-merge", "stitched-merge"])
def test_r1_decode_t64(stitched):
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} stitched={stitched}")
    L = build_layer(cfg, stitched=stitched)
    try:
        _run(L)
        # every token and every one of the T*k rows
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T))
        assert n == cfg.R
        # a second step on the other half of the double buffer gives the same bits
        y0 = L.y.clone()
        torch.cuda.synchronize()
        L.forward(half=1)
        L.synchronize()
        assert torch.equal(L.y, y0)
    finally:
        L.close()


def test_r1_decode_t64_remote_pool_on_host():
    """The remote share (192 experts, 16.9 GB) in pinned host memory: the routed pull crosses
    PCIe into the stitched half.  Every row and every token is checked."""
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} remote pool in pinned host memory")
    L = build_layer(cfg, stitched=True, remote_on_host=True)
    try:
        assert not L._remote_t.is_cuda and L._remote_t.is_pinned()
        _run(L)
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T))
        assert n == cfg.R
    finally:
        L.close()


def test_r1_decode_t64_device_routed_pull():
    """The R1 decode layer with the routed pull decided on the device (no count read-back):
    every row and token, and y bit-equal to the host-routed step."""
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} device-routed pull")
    L = build_layer(cfg, stitched=True)
    try:
        L.forward(half=0, remote="device")
        L.synchronize()
        _check_device_slot_map(cfg, L, 0)
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T))
        assert n == cfg.R
        y_dev = L.y.clone()
        torch.cuda.synchronize()
        L.forward(half=1, remote="routed")
        L.synchronize()
        assert torch.equal(L.y, y_dev)
    finally:
        L.close()


def test_r1_decode_t64_graph_replay():
    """The R1 decode step captured into one HIP graph per buffer half and replayed: every
    replay bit-equal to the eager step, and the replayed output checked against the oracle on
    every row and token."""
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} graph replay")
    L = build_layer(cfg, stitched=True, fused_gather=True)
    try:
        L.forward(half=0, remote="device")
        L.synchronize()
        y0 = L.y.clone()
        graphs = [L.capture_step(h) for h in range(2)]
        for r in range(4):
            L.y.fill_(float("nan"))
            torch.cuda.synchronize()
            graphs[r % 2].replay()
            torch.cuda.synchronize()
            assert torch.equal(L.y, y0), f"replay {r}"
        _check_device_slot_map(cfg, L, 1)
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T), check_xperm=False)
        assert n == cfg.R
        del graphs
    finally:
        L.close()


def test_r1_decode_t64_dwdp3_split():
    """The 3-rank split: 86 local experts, 170 fetched; stitched merge.  Every row and every
    token is checked."""
    cfg = synth.config("r1_decode_t64_dwdp3")
    log(f"case {cfg.name}")
    L = build_layer(cfg, stitched=True)
    try:
        _run(L)
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T))
        assert n == cfg.R
        assert L.last_ids[: cfg.n_local] == list(range(cfg.n_local))
    finally:
        L.close()


@pytest.mark.parametrize("stitched", [False, True], ids=["copy-merge", "stitched-merge"])
def test_r1_decode_t64_chunked_prefetch(stitched):
    """Remote fetch in 4 chunks with one ready event each; the GEMM runs per chunk.  Every
    row and every token is checked."""
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} chunks=4 stitched={stitched}")
    L = build_layer(cfg, stitched=stitched)
    try:
        L.forward(half=0, chunks=4)
        _, n = check_rows(cfg, L, range(cfg.R), range(cfg.T))
        assert n == cfg.R
        y0 = L.y.clone()
        torch.cuda.synchronize()
        L.forward(half=1, chunks=0)
        L.synchronize()
        assert torch.equal(L.y, y0)
    finally:
        L.close()


@pytest.mark.parametrize("chunks", [1, 3, 7])
def test_small_bf16_chunked_prefetch(chunks):
    cfg = synth.MoEConfig("bf16_chunks", T=50, H=136, I=72, E=37, k=3, dtype="bf16", n_local=9,
                          seed=1087)
    L = build_layer(cfg)
    L.forward(half=0, chunks=chunks)
    check_full(cfg, L)


@pytest.mark.parametrize("T,H,I,E,k,n_local", [
    (50, 136, 72, 37, 3, 9),       # decode tiles, ragged
    (300, 128, 64, 8, 2, 2),       # prefill tiles
    (64, 256, 512, 8, 2, 4),       # fp32 is covered below
])
def test_fused_gather_small(T, H, I, E, k, n_local):
    cfg = synth.MoEConfig(f"bf16_gather_T{T}", T=T, H=H, I=I, E=E, k=k, dtype="bf16",
                          n_local=n_local, seed=1000 + T + E)
    L = build_layer(cfg, fused_gather=True)
    L.forward(half=0)
    out = L.outputs()
    x = synth.activations(cfg)
    logits = synth.logits(cfg)
    check_routing(cfg, out, logits)
    ref = O.moe_layer(x, logits, cfg.k, weights_fn(L), cfg.H, cfg.I, round_h=True)
    assert rel_err(out["y"], ref["y"]) <= TOL["bf16"]
    assert rel_err(out["y_perm"], ref["y_perm"]) <= TOL["bf16"]


def test_fused_gather_tiny_fp32():
    cfg = synth.config("tiny_fp32_t64")
    L = build_layer(cfg, fused_gather=True)
    L.forward(half=0)
    out = L.outputs()
    ref = O.moe_layer(synth.activations(cfg), synth.logits(cfg), cfg.k, weights_fn(L), cfg.H, cfg.I,
                      round_h=False)
    assert rel_err(out["y"], ref["y"]) <= TOL["f32"]


def test_r1_prefill_t16384_fused_gather():
    """As bench.py runs it (stitched merge, gather on load, device-routed pull): every one of
    the 131072 rows of y_perm and every one of the 16384 tokens of y against the oracle."""
    cfg = synth.config("r1_prefill_t16384")
    log(f"case {cfg.name} fused gather, every row")
    L = build_layer(cfg, stitched=True, fused_gather=True)
    try:
        L.forward(half=0, remote="device")
        _, n = check_every_row(cfg, L, check_xperm=False)
        assert n == cfg.R
    finally:
        L.close()


def test_stitched_halves_small():
    """Both halves map the same local-expert block: merging copies nothing, results match."""
    from grouped_gemm_weights_amd import binding as B
    # a 1024 x 1024 expert block is 6 MiB, so the local and remote blocks are whole 2 MiB pages
    cfg = synth.MoEConfig("bf16_stitched", T=64, H=1024, I=1024, E=16, k=4, dtype="bf16",
                          n_local=4, seed=21)
    g = B.moe_vmm_granularity(0)
    if (cfg.n_local * synth.expert_block_bytes(cfg)) % g:
        pytest.skip(f"allocation granularity {g} does not divide the local block")
    L = build_layer(cfg, stitched=True, host_weights=True)
    try:
        _run(L)
        check_full(cfg, L)
        L.forward(half=1)
        check_full(cfg, L)
    finally:
        L.close()


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_r1_prefill_t8192_zipf(fused):
    """Skewed routing: a few experts with thousands of rows (full tiles), many with a handful
    (short tiles).  Every one of the 65536 rows of y_perm and every token of y, as bench.py
    runs it (stitched merge, gather on load, device-routed pull) and with x_perm built by
    moe_permute (checked bitwise) and the host-routed pull."""
    cfg = synth.config("r1_prefill_t8192_zipf")
    log(f"case {cfg.name} fused={fused}")
    L = build_layer(cfg, stitched=fused, fused_gather=fused)
    try:
        _run(L, remote="device" if fused else "routed")
        out, n = check_every_row(cfg, L, check_xperm=not fused)
        assert n == cfg.R
        log(f"active experts {int((out['counts'] > 0).sum())}, max rows {int(out['counts'].max())}")
    finally:
        L.close()


def test_r1_prefill_t16384():
    """Copy merge, x_perm built by moe_permute (checked bitwise), the whole remote share
    pulled: every row of y_perm and every token of y."""
    cfg = synth.config("r1_prefill_t16384")
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg), remote="all")
    _, n = check_every_row(cfg, L)
    assert n == cfg.R


# ----------------------------------------------------------------------------
# the combine folded into the down GEMM's epilogue (moe_grouped_swiglu_combine)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,I,E,k,n_local", [
    (50, 136, 72, 37, 3, 9),       # decode tiles, K and N tails
    (300, 128, 64, 8, 2, 2),       # prefill tiles, ragged tail
    (700, 256, 192, 12, 2, 3),     # full 256-row tiles and a partial column block
    (12, 1024, 200, 40, 6, 10),    # decode tiles, K = 1024
    (64, 256, 512, 8, 1, 4),       # k = 1
])
def test_combine_in_epilogue_small(T, H, I, E, k, n_local):
    """Every token's y against the oracle, and against the two-call path (grouped GEMM then
    moe_combine) to fp32 rounding: the atomics add a token's k rows in no fixed order."""
    cfg = synth.MoEConfig(f"bf16_comb_T{T}_E{E}_k{k}", T=T, H=H, I=I, E=E, k=k, dtype="bf16",
                          n_local=n_local, seed=3000 + T + E)
    log(f"case {cfg.name}")
    L = build_layer(cfg, combine_in_epilogue=True)
    L.forward(half=0)
    out = L.outputs()
    assert out["status"] == 0
    check_routing(cfg, out, synth.logits(cfg))
    ref = O.moe_layer(synth.activations(cfg), synth.logits(cfg), cfg.k, weights_fn(L), cfg.H,
                      cfg.I, True)
    e_y = rel_err(out["y"], ref["y"])
    L2 = build_layer(cfg, fused_gather=True)
    L2.forward(half=0)
    y2 = L2.outputs()["y"]
    e_2 = rel_err(out["y"], y2)
    log(f"{cfg.name}: y err/rms {e_y:.3e}; against the two-call path {e_2:.3e}")
    assert e_y <= TOL["bf16"]
    assert e_2 <= 1e-5
    if k == 1:
        # one term per token: the atomic adds w = 1.0 times the row to zero, exactly
        np.testing.assert_array_equal(out["y"], y2)


def test_combine_in_epilogue_r1_decode_t64():
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} combine in epilogue")
    L = build_layer(cfg, stitched=True, combine_in_epilogue=True)
    try:
        _run(L)
        check_y_tokens(cfg, L, range(cfg.T))
    finally:
        L.close()


def test_combine_in_epilogue_r1_prefill_t16384():
    cfg = synth.config("r1_prefill_t16384")
    log(f"case {cfg.name} combine in epilogue")
    L = build_layer(cfg, stitched=True, combine_in_epilogue=True)
    try:
        L.forward(half=0, remote="all")
        check_y_tokens(cfg, L, range(cfg.T))
    finally:
        L.close()


def test_debug_sync_mode(monkeypatch):
    """MOE_DEBUG_SYNC=1: every call synchronises; results are unchanged, and a status bit set
    by a call's kernels comes back from that very call as MOE_ERR_STATUS."""
    from grouped_gemm_weights_amd import binding as B
    cfg = synth.MoEConfig("bf16_debug_sync", T=80, H=128, I=64, E=12, k=3, dtype="bf16",
                          n_local=3, seed=41)
    log(f"case {cfg.name}")
    L = build_layer(cfg)
    L.forward(half=0)
    ref = L.outputs()
    monkeypatch.setenv("MOE_DEBUG_SYNC", "1")
    L.forward(half=1)
    out = L.outputs()
    assert out["status"] == 0
    assert out["y"].tobytes() == ref["y"].tobytes()
    logits = synth.logits(cfg)
    logits[3, 5] = np.nan
    L.set_inputs(synth.activations(cfg), logits)
    with pytest.raises(B.MoEError) as e:
        L.route_permute()
    assert e.value.code == B.MOE_ERR_STATUS
    assert "moe_route" in str(e.value) and "non-finite" in str(e.value)
