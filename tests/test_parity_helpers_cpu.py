"""The full-size GPU checks build their expected values from oracle pieces in parallel
(tests/moe_cases.py: expert_ffn_rows, tokens_layer, check_rows, check_every_row,
tile_boundary_rows).
These CPU tests pin those helpers: they agree with the oracle's own whole-layer and
per-token functions, select the rows they claim to, and fail on a planted wrong row."""
import numpy as np
import pytest

from moe_cases import (O, check_every_row, check_rows, expert_ffn_rows, synth, tile_boundary_rows,
                       tokens_layer)

torch = pytest.importorskip("torch")


def _cfg():
    return synth.MoEConfig("bf16_helpers", T=40, H=32, I=24, E=9, k=3, dtype="bf16", n_local=3,
                           seed=61, zipf_s=1.1, rho_seed=62)


def test_tokens_layer_equals_moe_layer_tokens():
    cfg = _cfg()
    x, L = synth.activations(cfg), synth.logits(cfg)
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    tok = [1, 2, 5, 17, 39]
    ref = O.moe_layer_tokens(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, True, tok)["y"]
    got = tokens_layer(lambda e: blocks[e], x[tok], L[tok], cfg.k, cfg.H, cfg.I, True, workers=3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_expert_ffn_rows_per_expert():
    cfg = _cfg()
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    rng = np.random.default_rng(3)
    rows = {e: rng.standard_normal((e + 1, cfg.H)) for e in (0, 4, 8)}
    got = expert_ffn_rows(lambda e: blocks[e], rows, cfg.H, cfg.I, True, workers=2)
    for e, xr in rows.items():
        wg, wu, wd = O.expert_matrices(blocks[e], cfg.H, cfg.I)
        np.testing.assert_array_equal(got[e], O.swiglu_ffn(xr, wg, wu, wd, True))


def test_tile_boundary_rows_cover_every_tile_edge():
    offsets = np.array([0, 0, 1, 33, 33, 600, 640])
    rows = set(tile_boundary_rows(offsets))
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            assert {lo, hi - 1} <= rows
        # any tile plan whose tiles are whole 32-row blocks (the last one excepted)
        for height in (64, 128, 192, 256, 288, 320):
            for t0 in range(lo, hi, height):
                assert t0 in rows and min(hi, t0 + height) - 1 in rows
    assert rows <= set(range(offsets[-1]))


class _FakeLayer:
    """Stands in for MoELayer: outputs() returns the oracle's own layer as a GPU would (f32)."""

    def __init__(self, cfg, perturb_row=None):
        self.cfg = cfg
        self.blocks = synth.pool_np(cfg, 0, range(cfg.E))
        ref = O.moe_layer(synth.activations(cfg), synth.logits(cfg), cfg.k,
                          lambda e: self.blocks[e], cfg.H, cfg.I, True)
        self.out = {k: ref[k] for k in ("idx", "w", "counts", "offsets", "row_of", "src_of",
                                        "x_perm")}
        self.out["y_perm"] = ref["y_perm"].astype(np.float32)
        if perturb_row is not None:
            rms = np.sqrt(np.mean(ref["y_perm"] ** 2))
            self.out["y_perm"][perturb_row, 3] += np.float32(0.1 * rms)
        self.out["y"] = ref["y"].astype(np.float32)
        self.out["status"] = 0

    def outputs(self):
        return self.out

    def expert_block(self, e):
        return torch.from_numpy(self.blocks[e].view(np.int16)).view(torch.bfloat16)


def test_check_rows_passes_on_oracle_outputs_and_catches_a_wrong_row():
    cfg = _cfg()
    check_rows(cfg, _FakeLayer(cfg), tile_boundary_rows, [0, 7, 39], workers=2)
    fake = _FakeLayer(cfg)
    offs = fake.out["offsets"]
    e = int(np.argmax(np.diff(offs)))
    bad_row = int(offs[e + 1] - 1)                   # the last row of the largest group
    with pytest.raises(AssertionError):
        check_rows(cfg, _FakeLayer(cfg, perturb_row=bad_row), tile_boundary_rows, [0], workers=2)


def test_check_every_row_passes_on_oracle_outputs_and_catches_a_wrong_row_or_token():
    cfg = _cfg()
    _, n = check_every_row(cfg, _FakeLayer(cfg), workers=3, row_block=7)
    assert n == cfg.R
    fake = _FakeLayer(cfg)
    offs = fake.out["offsets"]
    e = int(np.argmin(np.where(np.diff(offs) > 0, np.diff(offs), 10 ** 9)))
    # a middle row of the smallest group, away from any 32-row tile edge
    bad_row = int((offs[e] + offs[e + 1] - 1) // 2)
    with pytest.raises(AssertionError):
        check_every_row(cfg, _FakeLayer(cfg, perturb_row=bad_row), workers=3, row_block=7)
    bad = _FakeLayer(cfg)
    rms = np.sqrt(np.mean(bad.out["y"].astype(np.float64) ** 2))
    bad.out["y"][cfg.T // 2, 5] += np.float32(0.1 * rms)
    with pytest.raises(AssertionError):
        check_every_row(cfg, bad, workers=3, row_block=7)
