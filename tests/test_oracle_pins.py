"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks one oracle function against brute force on tiny inputs, a
library routine, a closed form or an invariant, chosen so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a
non-stable order) fails at least one of them.  The pages print no worked
example (see tests/golden/README.md), so none of the pins is a printed value.
"""
import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import moe as O  # noqa: E402
from grouped_gemm_weights_amd import synth  # noqa: E402


# ----------------------------------------------------------------------------
# brute-force helpers (pure Python; deliberately different algorithms)
# ----------------------------------------------------------------------------

def brute_topk(row, k):
    """k passes of 'take the largest remaining logit, lowest id on ties'."""
    taken = set()
    out = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.add(best)
        out.append(best)
    return out


def brute_permutation(flat, E):
    src = []
    for e in range(E):
        for a, v in enumerate(flat):
            if v == e:
                src.append(a)
    row = [0] * len(flat)
    for r, a in enumerate(src):
        row[a] = r
    return row, src


def brute_ffn_row(x, wg, wu, wd, round_h=None):
    """One token through one expert with explicit index loops (W stored out x in)."""
    H = len(x)
    I = len(wg)
    h = []
    for i in range(I):
        g = sum(x[c] * wg[i][c] for c in range(H))
        u = sum(x[c] * wu[i][c] for c in range(H))
        s = g / (1.0 + math.exp(-g))
        hv = s * u
        if round_h is not None:
            hv = round_h(hv)
        h.append(hv)
    return [sum(h[i] * wd[o][i] for i in range(I)) for o in range(H)]


# ----------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------

def test_round_to_bf16_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # fp32/bf16 subnormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_to_bf16_ties_and_specials():
    # bf16 spacing at 1.0 is 2**-7: a half-way value rounds to the even neighbour
    assert O.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert O.round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 1 + 2 ** -7
    assert O.round_to_bf16(np.array([-(1 + 2 ** -8)]))[0] == -1.0
    # subnormal spacing 2**-133
    assert O.round_to_bf16(np.array([2.0 ** -133 * 0.5]))[0] == 0.0          # tie -> even (0)
    assert O.round_to_bf16(np.array([2.0 ** -133 * 1.5]))[0] == 2.0 ** -132   # tie -> even (2)
    assert O.round_to_bf16(np.array([1e39]))[0] == np.inf


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3F81], dtype=np.uint16)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits),
                                  [1.0, -1.0, 2.0, 0.0, -0.0, 1 + 2 ** -7])


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 16, 5), (20, 33, 33), (30, 256, 8)])
def test_route_matches_bruteforce(T, E, k):
    rng = np.random.default_rng(T * E + k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[::3] = np.round(L[::3] * 2) / 2        # quantised rows force ties
    L[1, :] = 0.0
    L[1, ::2] = -0.0                          # +0 and -0 compare equal
    idx, w = O.route(L, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk(L[t].tolist(), k)
        ex = [math.exp(float(L[t, e]) - float(L[t, idx[t, 0]])) for e in idx[t]]
        s = sum(ex)
        np.testing.assert_allclose(w[t], [v / s for v in ex], rtol=1e-6, atol=0)


def test_route_equals_renormalised_full_softmax():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((64, 8)).astype(np.float32)
    idx, w = O.route(L, 2)
    full = np.exp(L.astype(np.float64))
    full /= full.sum(axis=1, keepdims=True)
    chosen = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, chosen / chosen.sum(axis=1, keepdims=True), rtol=1e-6)


def test_route_invariants_and_closed_forms():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((100, 32)).astype(np.float32)
    idx, w = O.route(L, 6)
    for t in range(100):
        assert len(set(idx[t])) == 6
        vals = L[t, idx[t]]
        assert np.all(np.diff(vals) <= 0)
        assert np.all(np.diff(w[t]) <= 0)
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 1)) <= 1e-6
    # k = 1 -> weight exactly 1
    i1, w1 = O.route(L, 1)
    assert np.all(w1 == 1.0)
    np.testing.assert_array_equal(i1[:, 0], np.argmax(L, axis=1))
    # all logits equal -> ids 0..k-1, weights 1/k
    ie, we = O.route(np.full((3, 10), 0.25, np.float32), 4)
    np.testing.assert_array_equal(ie, np.tile(np.arange(4), (3, 1)))
    np.testing.assert_allclose(we, 0.25, rtol=0, atol=0)
    # k = E -> the full stable descending order
    ik, _ = O.route(L[:5, :9], 9)
    for t in range(5):
        assert list(ik[t]) == sorted(range(9), key=lambda e: (-float(L[t, e]), e))
    # one-hot logits: the hot expert first, then ids ascending among the zeros
    oh = np.zeros((2, 6), np.float32)
    oh[0, 4] = 1.0
    oh[1, 0] = 1.0
    io, wo = O.route(oh, 3)
    np.testing.assert_array_equal(io, [[4, 0, 1], [0, 1, 2]])
    e1 = math.e
    np.testing.assert_allclose(wo[0], [e1 / (e1 + 2), 1 / (e1 + 2), 1 / (e1 + 2)], rtol=1e-7)


def test_route_rejects_nonfinite():
    L = np.zeros((2, 4), np.float32)
    L[1, 2] = np.nan
    with pytest.raises(ValueError):
        O.route(L, 2)
    L[1, 2] = np.inf
    with pytest.raises(ValueError):
        O.route(L, 2)


# ----------------------------------------------------------------------------
# counts, offsets, permutation, gather
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(17, 5, 2), (64, 8, 2), (9, 12, 12), (33, 256, 8)])
def test_counts_offsets_permutation_bruteforce(T, E, k):
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = O.route(L, k)
    flat = idx.ravel().tolist()
    counts = O.expert_counts(idx, E)
    assert counts.sum() == T * k
    for e in range(E):
        assert counts[e] == sum(1 for v in flat if v == e)
    offsets = O.expert_offsets(counts)
    assert offsets[0] == 0 and offsets[-1] == T * k
    for e in range(E):
        assert offsets[e + 1] - offsets[e] == counts[e]
    row_of, src_of = O.permutation(idx, E)
    br, bs = brute_permutation(flat, E)
    assert list(src_of) == bs and list(row_of) == br
    np.testing.assert_array_equal(np.sort(src_of), np.arange(T * k))
    np.testing.assert_array_equal(row_of[src_of], np.arange(T * k))
    for e in range(E):
        rows = src_of[offsets[e]:offsets[e + 1]]
        assert all(flat[a] == e for a in rows)
        assert list(rows) == sorted(rows)


def test_permutation_degenerate():
    idx = np.full((7, 1), 3, np.int32)          # all tokens on one expert
    row_of, src_of = O.permutation(idx, 5)
    np.testing.assert_array_equal(src_of, np.arange(7))
    np.testing.assert_array_equal(O.expert_offsets(O.expert_counts(idx, 5)), [0, 0, 0, 0, 7, 7])
    with pytest.raises(ValueError):
        O.permutation(np.array([[5]], np.int32), 5)


def test_gather_rows_bitwise():
    x = synth.to_bf16_bits(np.random.default_rng(1).standard_normal((6, 10)).astype(np.float32))
    src = np.array([5, 0, 11, 3, 3, 7, 1, 2, 4, 6, 8, 9, 10, 0][:12], np.int32)
    xp = O.gather_rows(x, src, 2)
    for r, a in enumerate(src):
        assert xp[r].tobytes() == x[a // 2].tobytes()


# ----------------------------------------------------------------------------
# merge
# ----------------------------------------------------------------------------

def test_slot_map_and_merge_bruteforce():
    rng = np.random.default_rng(2)
    local = rng.integers(0, 65535, size=(4, 12), dtype=np.uint16)
    remote = rng.integers(0, 65535, size=(4, 12), dtype=np.uint16)
    ids = [0, 1, 2, 3, 5, 7]
    s = O.slot_map(ids, 8)
    assert list(s) == [0, 1, 2, 3, -1, 4, -1, 5]
    m = O.merge([(0, local), (4, remote)], ids)
    for e in range(8):
        if s[e] >= 0:
            src = local[e] if e < 4 else remote[e - 4]
            assert m[s[e]].tobytes() == src.tobytes()
    with pytest.raises(ValueError):
        O.slot_map([3, 1], 8)
    with pytest.raises(ValueError):
        O.merge([(0, local), (4, remote)], [8])


# ----------------------------------------------------------------------------
# SwiGLU experts
# ----------------------------------------------------------------------------

def test_silu_closed_forms():
    scipy_special = pytest.importorskip("scipy.special")
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z), z * scipy_special.expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(np.array([2.0]))[0], 2 / (1 + math.exp(-2)), rtol=1e-15)


def test_expert_layout_and_ffn_bruteforce():
    H, I = 6, 4
    rng = np.random.default_rng(5)
    blk = rng.standard_normal(3 * H * I)
    wg, wu, wd = O.expert_matrices(blk, H, I)
    # layout: [Wg I x H][Wu I x H][Wd H x I], row-major, out x in
    assert wg[2, 5] == blk[2 * H + 5]
    assert wu[1, 0] == blk[H * I + 1 * H]
    assert wd[5, 3] == blk[2 * H * I + 5 * I + 3]
    x = rng.standard_normal((3, H))
    got = O.swiglu_ffn(x, wg, wu, wd, round_h=False)
    for r in range(3):
        ref = brute_ffn_row(x[r].tolist(), wg.tolist(), wu.tolist(), wd.tolist())
        np.testing.assert_allclose(got[r], ref, rtol=1e-12, atol=1e-14)
    # with bf16 storage of h, against the torch cast of each h value
    torch = pytest.importorskip("torch")

    def rh(v):
        return float(torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64))
    got_r = O.swiglu_ffn(x, wg, wu, wd, round_h=True)
    for r in range(3):
        ref = brute_ffn_row(x[r].tolist(), wg.tolist(), wu.tolist(), wd.tolist(), round_h=rh)
        np.testing.assert_allclose(got_r[r], ref, rtol=1e-12, atol=1e-14)


def test_ffn_zero_gate_and_single_expert_dense():
    H, I = 16, 8
    rng = np.random.default_rng(9)
    wg, wu, wd = (rng.standard_normal((I, H)), rng.standard_normal((I, H)),
                  rng.standard_normal((H, I)))
    x = rng.standard_normal((5, H))
    assert np.all(O.swiglu_ffn(x, np.zeros_like(wg), wu, wd, False) == 0.0)
    assert np.all(O.swiglu_ffn(x, wg, np.zeros_like(wu), wd, False) == 0.0)
    # E = 1, k = 1: the layer is one dense SwiGLU FFN with weight exactly 1
    blk = np.concatenate([wg.ravel(), wu.ravel(), wd.ravel()])
    res = O.moe_layer(x, np.zeros((5, 1), np.float32), 1, lambda e: blk, H, I, round_h=False)
    g = np.einsum("th,ih->ti", x, wg)
    u = np.einsum("th,ih->ti", x, wu)
    dense = np.einsum("ti,hi->th", g * (1 / (1 + np.exp(-g))) * u, wd)
    np.testing.assert_allclose(res["y"], dense, rtol=1e-12, atol=1e-13)


def test_combine_bruteforce_and_k1_exact():
    rng = np.random.default_rng(4)
    T, k, H = 6, 3, 5
    yp = rng.standard_normal((T * k, H)).astype(np.float32)
    row_of = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = O.combine(yp, row_of, w, k)
    for t in range(T):
        for h in range(H):
            ref = 0.0
            for j in range(k):
                ref += float(w[t, j]) * float(yp[row_of[t * k + j], h])
            assert abs(y[t, h] - ref) <= 1e-12
    y1 = O.combine(yp[:T], row_of[:T] % T, np.ones((T, 1), np.float32), 1)
    np.testing.assert_array_equal(y1, yp[:T][row_of[:T] % T].astype(np.float64))


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def dense_bruteforce_layer(x, L, k, blocks, H, I, round_h):
    """Every expert on every token, weighted by a gate that is 0 for unchosen experts.

    The routing weights are stored as float32 (the routing output format), so
    the gate takes the float32 value of each weight.
    """
    T, E = L.shape
    gate = np.zeros((T, E))
    for t in range(T):
        ids = brute_topk(L[t].tolist(), k)
        ex = [math.exp(float(L[t, e]) - float(L[t, ids[0]])) for e in ids]
        for e, v in zip(ids, ex):
            gate[t, e] = float(np.float32(v / sum(ex)))
    xd = O.decode(x)
    y = np.zeros((T, H))
    for e in range(E):
        d = O.decode(blocks[e])
        wg = d[: H * I].reshape(I, H)
        wu = d[H * I: 2 * H * I].reshape(I, H)
        wd = d[2 * H * I:].reshape(H, I)
        g = xd @ wg.T
        h = g / (1 + np.exp(-g)) * (xd @ wu.T)
        if round_h:
            h = O.round_to_bf16(h)
        y += gate[:, e:e + 1] * (h @ wd.T)
    return y


def test_layer_tiny_fp32_config_dense_bruteforce():
    cfg = synth.config("tiny_fp32_t64")
    x = synth.activations(cfg)
    L = synth.logits(cfg)
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    res = O.moe_layer(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, round_h=False)
    ref = dense_bruteforce_layer(x, L, cfg.k, blocks, cfg.H, cfg.I, False)
    assert np.max(np.abs(res["y"] - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))
    # sampled per-token path agrees with the permuted path
    tok = [0, 5, 17, 63]
    rt = O.moe_layer_tokens(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, False, tok)
    np.testing.assert_allclose(rt["y"], res["y"][tok], rtol=1e-12, atol=1e-12)
    # layer-output scale sanity: top-2 of 8 with unit-variance inputs
    assert 0.05 < np.sqrt(np.mean(ref ** 2)) < 5


def test_layer_bf16_small_dense_bruteforce():
    cfg = synth.MoEConfig("bf16_small", T=24, H=32, I=16, E=10, k=3, dtype="bf16",
                          n_local=3, seed=77, zipf_s=1.1, rho_seed=78)
    x = synth.activations(cfg)
    L = synth.logits(cfg)
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    res = O.moe_layer(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, round_h=True)
    ref = dense_bruteforce_layer(x, L, cfg.k, blocks, cfg.H, cfg.I, True)
    assert np.max(np.abs(res["y"] - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))
    # the h rounding is a small perturbation of the unrounded definition
    unr = dense_bruteforce_layer(x, L, cfg.k, blocks, cfg.H, cfg.I, False)
    rel = np.max(np.abs(ref - unr)) / np.sqrt(np.mean(unr ** 2))
    assert 0 < rel < 2e-2


def test_pipeline_two_layers_bruteforce():
    cfg = synth.MoEConfig("pipe_small", T=12, H=16, I=8, E=6, k=2, dtype="bf16",
                          n_local=2, seed=91, layers=2, dense_standin=True)
    x0 = synth.activations(cfg, 0)
    specs = []
    for l in range(2):
        blocks = synth.pool_np(cfg, l, range(cfg.E))
        specs.append(dict(logits=synth.logits(cfg, l), w_attn=synth.dense_weight_np(cfg, l),
                          weights_of=(lambda b: (lambda e: b[e]))(blocks), blocks=blocks))
    out = O.pipeline(x0, specs, cfg.k, cfg.H, cfg.I)
    x = O.decode(x0)
    for l, s in enumerate(specs):
        a = O.round_to_bf16(x @ O.decode(s["w_attn"]).T)
        y = dense_bruteforce_layer(a, s["logits"], cfg.k, s["blocks"], cfg.H, cfg.I, True)
        xn = O.round_to_bf16(x + y)
        np.testing.assert_allclose(out[l]["y"], y, rtol=1e-11, atol=1e-12)
        np.testing.assert_array_equal(out[l]["x_out"], xn)
        x = xn


# ----------------------------------------------------------------------------
# input generators: deterministic, shaped as documented
# ----------------------------------------------------------------------------

def test_synth_determinism_and_stats():
    cfg = synth.config("tiny_fp32_t64")
    assert synth.digest(synth.logits(cfg)) == synth.digest(synth.logits(cfg))
    b = synth.expert_block_np(cfg, 0, 3)
    H, I = cfg.H, cfg.I
    assert abs(np.std(b[: 2 * H * I]) * math.sqrt(H) - 1) < 0.02
    assert abs(np.std(b[2 * H * I:]) * math.sqrt(I) - 1) < 0.02
    z = synth.config("r1_prefill_t8192_zipf").with_(T=512)
    idx, _ = O.route(synth.logits(z), z.k)
    c = O.expert_counts(idx, z.E)
    assert c.max() > 0.8 * z.T            # one hot expert takes most tokens
    assert (c > 0).sum() < z.E            # skew leaves experts idle


# ----------------------------------------------------------------------------
# pipeline blocks: dense stand-in and residual, against index loops with an
# independent rounding to bf16 (exact rational arithmetic, not the oracle's
# frexp/rint route)
# ----------------------------------------------------------------------------

def brute_bf16(v):
    """Nearest bf16 value of a float by exact rational comparison of its two neighbours,
    ties to the one with an even last significand bit (normal range only)."""
    from fractions import Fraction
    if v == 0.0:
        return v
    m, e = math.frexp(abs(v))                 # |v| = m 2^e, m in [0.5, 1)
    step = Fraction(2) ** (e - 8)             # bf16 keeps 8 significant bits
    q = Fraction(abs(v)) / step
    lo = math.floor(q)
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return math.copysign(float(lo * step), v)


def test_brute_bf16_agrees_with_torch_cast():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(5).standard_normal(3000).astype(np.float32) * 7
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert [brute_bf16(float(a)) for a in v] == ref.tolist()


def test_dense_standin_index_loops():
    """A = bf16(x W^T) with W stored out x in, W deliberately not symmetric."""
    rng = np.random.default_rng(41)
    M, H = 5, 12
    x = synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w = synth.to_bf16_bits((rng.standard_normal((H, H)) / math.sqrt(H)).astype(np.float32))
    xd, wd = O.decode(x).tolist(), O.decode(w).tolist()
    want = [[brute_bf16(sum(xd[m][c] * wd[n][c] for c in range(H))) for n in range(H)]
            for m in range(M)]
    got = O.dense_standin(x, w)
    np.testing.assert_array_equal(got, np.array(want))
    # the stand-in output lies on the bf16 grid
    np.testing.assert_array_equal(O.round_to_bf16(got), got)


def test_residual_index_loops():
    """x_next = bf16(x + y): x bf16 bits, y float32, one rounding of the exact sum."""
    rng = np.random.default_rng(43)
    x = synth.to_bf16_bits(rng.standard_normal((4, 9)).astype(np.float32))
    y = (rng.standard_normal((4, 9)) * 0.3).astype(np.float32)
    y[0, 0] = 2.0 ** -9                           # x + y lands next to a rounding boundary
    xd = O.decode(x)
    want = [[brute_bf16(float(xd[i, j]) + float(y[i, j])) for j in range(9)] for i in range(4)]
    np.testing.assert_array_equal(O.residual(x, y), np.array(want))


def test_layer_tokens_round_h_matches_dense_bruteforce():
    """The per-token path with the bf16 h rounding (the path the full-size GPU checks use)
    against the dense every-expert evaluation with the same rounding."""
    cfg = synth.MoEConfig("bf16_small_tok", T=24, H=32, I=16, E=10, k=3, dtype="bf16",
                          n_local=3, seed=79, zipf_s=1.1, rho_seed=80)
    x = synth.activations(cfg)
    L = synth.logits(cfg)
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    ref = dense_bruteforce_layer(x, L, cfg.k, blocks, cfg.H, cfg.I, True)
    tok = [0, 3, 7, 11, 23]
    rt = O.moe_layer_tokens(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, True, tok)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(rt["y"] - ref[tok])) <= 1e-12 * scale
    # and without the rounding it is the unrounded definition, a measurably different value
    unr = dense_bruteforce_layer(x, L, cfg.k, blocks, cfg.H, cfg.I, False)
    assert np.max(np.abs(unr[tok] - ref[tok])) > 1e-6 * scale


# ----------------------------------------------------------------------------
# the bulk float32 path (the CPU baseline) against the float64 definition
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_fp32_t64", "bf16_small"])
def test_bulk_float32_path_matches_the_definition(name):
    if name == "tiny_fp32_t64":
        cfg = synth.config(name)
    else:
        cfg = synth.MoEConfig(name, T=48, H=64, I=40, E=12, k=4, dtype="bf16", n_local=3, seed=83)
    x, L = synth.activations(cfg), synth.logits(cfg)
    blocks = synth.pool_np(cfg, 0, range(cfg.E))
    rh = cfg.dtype == "bf16"
    ref = O.moe_layer(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, rh)
    got = O.moe_layer(x, L, cfg.k, lambda e: blocks[e], cfg.H, cfg.I, rh, dtype=np.float32)
    for key in ("idx", "w", "counts", "offsets", "row_of", "src_of"):
        np.testing.assert_array_equal(got[key], ref[key])
    assert got["y"].dtype == np.float32 and got["y_perm"].dtype == np.float32
    rms = np.sqrt(np.mean(ref["y"] ** 2))
    # float32 products over H terms; with h rounded to bf16 an element of h may land on the
    # other side of a rounding boundary (one bf16 spacing), which the 2e-2 bound absorbs
    tol = 1e-5 if not rh else 2e-2
    assert np.max(np.abs(got["y"] - ref["y"])) <= tol * rms
    assert np.max(np.abs(got["y"] - ref["y"])) > 0          # it really ran in float32
