"""GPU parity of the multi-layer pipelines (R1 shape, dense stand-in block per
layer, copy-stream prefetch into the double buffer): 6 layers of 4096 tokens
(copy and stitched merge) and 4 layers of 16384 tokens (stitched merge, fused
gather, as bench.py runs it).

Per layer, the oracle is fed the GPU's own layer input (bf16), as the layer
outputs are then compared one layer at a time; routing is checked bit-exactly
on all tokens; the dense block, the MoE output and the residual are checked on
sampled tokens.  Tokens are independent through every block, so the oracle
also runs the whole pipeline for the sampled tokens from the seeded
input and the final residual stream is compared end to end.

The dense block output and the residual stream are stored in bf16 on both
sides, so those comparisons allow one bf16 spacing of the reference per
element before applying the 2e-2 x RMS bound (rel_err_bf16); the MoE output
y is f32 and uses the plain bound.  End to end, the residual stream has been
rounded to bf16 once per layer, so one spacing per layer is allowed, and the
normwise error must also stay under 2e-2.
"""
import gc

import numpy as np
import pytest

from moe_cases import O, TOL, W_TOL, log, rel_err, rel_err_bf16, synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("stitched", [True, False], ids=["stitched-merge", "copy-merge"])
def test_r1_pipeline_6x4096(stitched):
    from grouped_gemm_weights_amd.layer import block_to_numpy
    from grouped_gemm_weights_amd.pipeline import MoEPipeline
    cfg = synth.config("r1_pipeline_6x4096")
    log(f"case {cfg.name} stitched={stitched}")
    P = MoEPipeline(cfg, stitched=stitched)
    try:
        _check_pipeline(cfg, P, block_to_numpy)
    finally:
        P.close()
        del P
        gc.collect()
        torch.cuda.empty_cache()


def test_r1_pipeline_4x16384():
    """Four layers at 16384 tokens each, stitched merge: the same checks as above."""
    from grouped_gemm_weights_amd.layer import block_to_numpy
    from grouped_gemm_weights_amd.pipeline import MoEPipeline
    cfg = synth.config("r1_pipeline_4x16384")
    log(f"case {cfg.name} stitched=True")
    P = MoEPipeline(cfg, stitched=True, fused_gather=True)
    try:
        _check_pipeline(cfg, P, block_to_numpy)
    finally:
        P.close()
        del P
        gc.collect()
        torch.cuda.empty_cache()


def _check_pipeline(cfg, P, block_to_numpy):
    tokens = sorted(np.random.default_rng(6).choice(cfg.T, size=4, replace=False).tolist())
    cap = []

    def hook(l):
        P.synchronize()
        cap.append(dict(x=_bits(P.x), a=_bits(P.a), y=P.L.y.detach().cpu().numpy(),
                        idx=P.L.topk_idx.cpu().numpy(), w=P.L.topk_w.cpu().numpy(),
                        counts=P.L.counts.cpu().numpy()))

    P.forward(layer_hook=hook)
    P.synchronize()
    assert P.L.read_status() == 0
    x_final = _bits(P.x)
    specs = []
    for l in range(cfg.layers):
        c = cap[l]
        logits = synth.logits(cfg, l)
        idx, w = O.route(logits, cfg.k)
        np.testing.assert_array_equal(c["idx"], idx)
        assert np.max(np.abs(c["w"].astype(np.float64) - w)) <= W_TOL
        np.testing.assert_array_equal(c["counts"], O.expert_counts(idx, cfg.E))
        w_attn = _bits(P.w_attn[l])

        def weights_of(e, l=l):
            blk = P.locals[l][e] if e < cfg.n_local else P.remotes[l][e - cfg.n_local]
            return block_to_numpy(blk)
        # dense stand-in on the GPU's own x_l
        a_ref = O.dense_standin(c["x"][tokens], w_attn)
        e_a = rel_err_bf16(O.decode(c["a"][tokens]), a_ref)
        # MoE block on the GPU's own A_l
        ref = O.moe_layer_tokens(c["a"], logits, cfg.k, weights_of, cfg.H, cfg.I, True, tokens)
        e_y = rel_err(c["y"][tokens], ref["y"])
        # residual on the GPU's own x_l and y_l: round to nearest bf16 of the sum
        x_next = cap[l + 1]["x"] if l + 1 < cfg.layers else x_final
        res_ref = O.residual(c["x"][tokens], c["y"][tokens])
        e_r = rel_err_bf16(O.decode(x_next[tokens]), res_ref)
        log(f"layer {l}: dense err/rms {e_a:.2e}, moe err/rms {e_y:.2e}, residual err/rms {e_r:.2e}")
        assert e_a <= TOL["bf16"] and e_y <= TOL["bf16"] and e_r <= TOL["bf16"]
        specs.append(dict(logits=logits[tokens], w_attn=w_attn, weights_of=weights_of))
    # end to end from the seeded input, oracle only
    x0 = synth.activations(cfg, 0)[tokens]
    out = O.pipeline(x0, specs, cfg.k, cfg.H, cfg.I)
    ref_end = out[-1]["x_out"]
    got_end = O.decode(x_final[tokens])
    # the residual stream is re-rounded to bf16 after every layer: one boundary per layer
    e_end = rel_err_bf16(got_end, ref_end, roundings=cfg.layers)
    norm_end = float(np.sqrt(np.mean((got_end - ref_end) ** 2) / np.mean(ref_end ** 2)))
    log(f"end-to-end after {cfg.layers} layers: err/rms beyond {cfg.layers} bf16 spacings {e_end:.2e}, "
        f"normwise {norm_end:.2e}")
    assert e_end <= TOL["bf16"] and norm_end <= TOL["bf16"]


def test_pipeline_event_timeline():
    """The per-layer schedule (explainer, prefetch-schedule and per-layer latency panels) read
    off the events of a pipelined pass over the 6 x 4096 workload: MoE block l starts only
    after layer l's copy has ended; the stall measured around the wait matches the copy
    timeline; copies are serial on their stream; a half is refilled only after the layer that
    read it (two layers back) has finished; and layer latency covers the layer's compute."""
    from grouped_gemm_weights_amd import binding as B
    from grouped_gemm_weights_amd.pipeline import MoEPipeline
    cfg = synth.config("r1_pipeline_6x4096")
    log(f"case {cfg.name} event timeline")
    P = MoEPipeline(cfg, stitched=True, fused_gather=True)
    n = cfg.layers
    keys = ("c0", "c1", "wait0", "wait1", "d0", "m1", "g1")
    evs = []
    try:
        P.forward()                                   # warm-up
        for _ in range(2):
            ev = {k: [B.moe_event_create(True) for _ in range(n)] for k in keys}
            evs.append(ev)
            P.forward(ev)
        P.synchronize()
        assert P.L.read_status() == 0
        tol = 0.05                                    # ms: event signalling across streams
        for ev in evs:
            t = lambda a, la, b, lb: B.moe_event_elapsed_ms(ev[a][la], ev[b][lb])
            for l in range(n):
                assert t("c1", l, "wait1", l) >= -tol, f"layer {l} ran before its weights landed"
                stall = t("wait0", l, "wait1", l)
                expect = max(0.0, t("wait0", l, "c1", l))
                assert abs(stall - expect) <= 2 * tol, (l, stall, expect)
                if l + 1 < n:
                    assert t("c1", l, "c0", l + 1) >= -tol, f"copies of layers {l}, {l + 1} overlap"
                if l >= 1 and l + 1 < n:
                    assert t("m1", l - 1, "c0", l + 1) >= -tol, f"half refilled while layer {l - 1} read it"
                if l >= 1:
                    assert t("m1", l - 1, "m1", l) >= t("d0", l, "m1", l) - tol
            lat = [t("m1", l - 1, "m1", l) for l in range(1, n)]
            log("layer latency " + ", ".join(f"{v:.2f}" for v in lat) + " ms")
    finally:
        for ev in evs:
            for lst in ev.values():
                for e in lst:
                    B.moe_event_destroy(e)
        P.close()
        del P
        gc.collect()
        torch.cuda.empty_cache()
