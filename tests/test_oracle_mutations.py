"""The pins must catch plausible mistakes: each case plants one in the oracle (CPU only).

Every mutation below replaces one oracle function with a subtly wrong variant
(dropped term, wrong sign, wrong index, transposed operand, unstable order)
and checks that at least one pin of ``test_oracle_pins`` then fails.
"""
import numpy as np
import pytest

from oracle import moe as O
import test_oracle_pins as P


def _wrong_silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))                      # sign flipped in the exponent


def _wrong_route_full_softmax(logits, k):
    L = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(L)):
        raise ValueError("non-finite router logit")
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int32)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)                      # not renormalised over the k
    return idx, np.take_along_axis(p, idx, 1).astype(np.float32)


def _wrong_route_tie(logits, k):
    L = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(L)):
        raise ValueError("non-finite router logit")
    idx = np.empty((L.shape[0], k), np.int32)
    w = np.empty((L.shape[0], k), np.float32)
    for t in range(L.shape[0]):
        order = np.argsort(-L[t][::-1], kind="stable")[:k]
        order = L.shape[1] - 1 - order                 # ties broken towards the larger id
        ex = np.exp(L[t, order] - L[t, order[0]])
        idx[t], w[t] = order, ex / ex.sum()
    return idx, w


def _wrong_permutation(idx, E):
    flat = np.asarray(idx).ravel()
    src_of = np.argsort(flat, kind="quicksort")[::-1].astype(np.int32)   # not stable
    src_of = src_of[np.argsort(flat[src_of], kind="stable")]
    row_of = np.empty_like(src_of)
    row_of[src_of] = np.arange(src_of.size, dtype=np.int32)
    return row_of, src_of


def _wrong_gather(x, src_of, k):
    return np.asarray(x)[np.asarray(src_of) % np.asarray(x).shape[0]].copy()   # % instead of //


def _wrong_matrices(block, H, I):
    wg, wu, wd = _orig["expert_matrices"](block, H, I)
    return wu, wg, wd                                   # gate and up swapped


def _wrong_ffn_transposed(x_rows, wg, wu, wd, round_h):
    x = O.decode(x_rows)
    g = x @ wg.T
    u = x @ wu.T
    h = O.silu(g) * u
    if round_h:
        h = O.round_to_bf16(h)
    return h @ wd.reshape(wd.shape[1], wd.shape[0])     # Wd read in the wrong layout


def _wrong_combine(y_perm, row_of, w, k):
    yp = np.asarray(y_perm, dtype=np.float64)
    T = np.asarray(w).shape[0]
    y = np.zeros((T, yp.shape[1]))
    for j in range(k):
        y += np.asarray(w, np.float64)[:, :1] * yp[np.asarray(row_of)[np.arange(T) * k + j]]   # w[t,0] for all j
    return y


def _wrong_round(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.trunc(v / q) * q                          # truncation instead of nearest-even


def _wrong_offsets(counts):
    return np.concatenate([np.cumsum(counts), [int(np.sum(counts))]]).astype(np.int32)   # inclusive scan


def _wrong_dense_transposed(x, w_attn):
    return O.round_to_bf16(O.decode(x) @ O.decode(w_attn))          # W used as in x out


def _wrong_dense_unrounded(x, w_attn):
    return O.decode(x) @ O.decode(w_attn).T                         # bf16 rounding dropped


def _wrong_residual_unrounded(x, y):
    return O.decode(x) + np.asarray(y, dtype=np.float64)            # bf16 rounding dropped


def _wrong_residual_y_rounded(x, y):
    return O.round_to_bf16(O.decode(x) + O.round_to_bf16(y))       # y rounded before the add


def _wrong_tokens_no_round_h(x, logits, k, weights_of, H, I, round_h, tokens):
    return _orig["moe_layer_tokens"](x, logits, k, weights_of, H, I, False, tokens)   # round_h dropped


_orig = {name: getattr(O, name) for name in
         ["silu", "route", "permutation", "gather_rows", "expert_matrices", "swiglu_ffn",
          "combine", "round_to_bf16", "expert_offsets", "dense_standin", "residual",
          "moe_layer_tokens"]}

MUTATIONS = [
    ("silu", _wrong_silu),
    ("route", _wrong_route_full_softmax),
    ("route", _wrong_route_tie),
    ("permutation", _wrong_permutation),
    ("gather_rows", _wrong_gather),
    ("expert_matrices", _wrong_matrices),
    ("swiglu_ffn", _wrong_ffn_transposed),
    ("combine", _wrong_combine),
    ("round_to_bf16", _wrong_round),
    ("expert_offsets", _wrong_offsets),
    ("dense_standin", _wrong_dense_transposed),
    ("dense_standin", _wrong_dense_unrounded),
    ("residual", _wrong_residual_unrounded),
    ("residual", _wrong_residual_y_rounded),
    ("moe_layer_tokens", _wrong_tokens_no_round_h),
]

PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_")]


def _run_pins():
    """Run every parametrisation-free pin plus the parametrised ones at one setting."""
    failures = 0
    for fn in PINS:
        params = {
            "test_route_matches_bruteforce": [(50, 8, 2), (30, 256, 8)],
            "test_counts_offsets_permutation_bruteforce": [(17, 5, 2), (33, 256, 8)],
            "test_bulk_float32_path_matches_the_definition": [("tiny_fp32_t64",), ("bf16_small",)],
        }.get(fn.__name__, [()])
        for args in params:
            try:
                fn(*args)
            except (Exception, pytest.fail.Exception):
                failures += 1
    return failures


def test_pins_pass_on_the_oracle():
    assert _run_pins() == 0


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_pins_catch_mutation(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    assert _run_pins() > 0, f"no pin caught the planted mistake in {name}"
