"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every test runs the library on seeded inputs and compares with the oracle
element by element: bit-exact for routing ids, counts, offsets, the
permutation and the gathered rows; within the tolerances of tests/moe_cases.py
for the routing weights and the float outputs.  Shapes span several tiles
with ragged tails; the DeepSeek-R1-shaped workloads run at full size with the
float outputs checked on sampled tokens.
"""
import gc

import numpy as np
import pytest

from moe_cases import (O, TOL, build_layer, check_full, check_routing, check_sampled, log,
                       rel_err, synth, weights_fn)

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


@pytest.mark.parametrize("fused", [False, True], ids=["x_perm", "fused-gather"])
def test_prefill_tile_modes_at_row_boundaries(fused):
    """Expert row counts on both sides of every prefill tile mode (64/128/192-row column-split
    tiles, full 256-row tiles, and a full tile plus a one-row tail), k = 1 so each count is
    exact; I = 192 leaves the gate/up GEMM a partial column block, so the epilogue runs both
    its unchecked (whole waves) and checked stores."""
    counts = [64, 65, 128, 129, 192, 193, 256, 257]
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


def test_injected_prefetch_fault_surfaces_and_recovers(monkeypatch):
    """MOE_INJECT_FAULT=prefetch: the layer step raises the library's error instead of running
    the GEMM on a half that was never filled; without it the next step is correct."""
    from grouped_gemm_weights_amd import binding as B
    cfg = synth.MoEConfig("bf16_fault", T=64, H=128, I=64, E=12, k=3, dtype="bf16", n_local=3,
                          seed=27)
    log(f"case {cfg.name}")
    L = build_layer(cfg)
    monkeypatch.setenv("MOE_INJECT_FAULT", "prefetch")
    with pytest.raises(B.MoEError) as e:
        L.forward(half=0)
    assert e.value.code == B.MOE_ERR_HIP
    monkeypatch.delenv("MOE_INJECT_FAULT")
    L.synchronize()
    L.forward(half=0)
    check_full(cfg, L)


def test_remote_pool_in_pinned_host_memory():
    cfg = synth.MoEConfig("bf16_host_remote", T=48, H=128, I=64, E=16, k=4, dtype="bf16",
                          n_local=4, seed=9)
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg, remote_on_host=True))
    check_full(cfg, L)


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


# ----------------------------------------------------------------------------
# DeepSeek-R1-shaped workloads at full size
# ----------------------------------------------------------------------------

def _sample(T, n, seed):
    return sorted(np.random.default_rng(seed).choice(T, size=n, replace=False).tolist())


@pytest.mark.parametrize("stitched", [False, True], ids=["copy-merge", "stitched-merge"])
def test_r1_decode_t64(stitched):
    cfg = synth.config("r1_decode_t64")
    log(f"case {cfg.name} stitched={stitched}")
    L = build_layer(cfg, stitched=stitched)
    try:
        _run(L)
        check_sampled(cfg, L, _sample(cfg.T, 8, 1))
        # a second step on the other half of the double buffer gives the same bits
        y0 = L.y.clone()
        torch.cuda.synchronize()
        L.forward(half=1)
        L.synchronize()
        assert torch.equal(L.y, y0)
    finally:
        L.close()


def test_r1_decode_t64_dwdp3_split():
    """The 3-rank split: 86 local experts, 170 fetched; stitched merge."""
    cfg = synth.config("r1_decode_t64_dwdp3")
    L = build_layer(cfg, stitched=True)
    try:
        _run(L)
        out = check_sampled(cfg, L, _sample(cfg.T, 4, 5))
        assert L.last_ids[: cfg.n_local] == list(range(cfg.n_local))
    finally:
        L.close()


@pytest.mark.parametrize("stitched", [False, True], ids=["copy-merge", "stitched-merge"])
def test_r1_decode_t64_chunked_prefetch(stitched):
    """Remote fetch in 4 chunks with one ready event each; the GEMM runs per chunk."""
    cfg = synth.config("r1_decode_t64")
    L = build_layer(cfg, stitched=stitched)
    try:
        L.forward(half=0, chunks=4)
        check_sampled(cfg, L, _sample(cfg.T, 4, 11))
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
    cfg = synth.config("r1_prefill_t16384")
    L = build_layer(cfg, stitched=True, fused_gather=True)
    try:
        L.forward(half=0, remote="all")
        check_sampled(cfg, L, _sample(cfg.T, 4, 13), check_xperm=False)
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


def test_r1_prefill_t8192_zipf():
    cfg = synth.config("r1_prefill_t8192_zipf")
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg))
    out = check_sampled(cfg, L, _sample(cfg.T, 6, 2))
    log(f"active experts {int((out['counts'] > 0).sum())}, max rows {int(out['counts'].max())}")


def test_r1_prefill_t16384():
    cfg = synth.config("r1_prefill_t16384")
    log(f"case {cfg.name}")
    L = _run(build_layer(cfg), remote="all")
    check_sampled(cfg, L, _sample(cfg.T, 6, 3))
