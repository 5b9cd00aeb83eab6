"""CPU oracle of the DWDP-style MoE layer forward.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and shares no code with
it; the two meet only at the seeded inputs of
``grouped_gemm_weights_amd.synth``.

Plain, slow, obviously correct numpy.  Floating point runs in float64; the
only rounding modelled is the one the workload fixes (bf16 storage of the
SwiGLU activation, see ``swiglu_ffn``).  No blocking, fusion or reordering
beyond what each definition states.

What the method computes (sources):

* The pages fix the system pattern: ranks stay data-parallel and hold a share
  of the MoE experts; missing ("remote") experts are pulled from peers on a
  copy engine into an alternate buffer one layer ahead (DWDP explainer, "stay
  data-parallel" and prefetch-schedule panels; DWDP arXiv 2604.01621v1,
  abstract), and local plus remote weights reach the grouped GEMM as one
  contiguous buffer (DWDP explainer, contiguous-buffer panel).
* The pages do not define the MoE layer itself.  Its plain definition is the
  top-k softmax-gated mixture of SwiGLU experts: route each token to its k
  largest router logits, renormalise the softmax over those k, run each
  chosen expert's SwiGLU FFN (Shazeer 2020, "GLU Variants Improve
  Transformer": silu on the gate projection, times the up projection, then
  the down projection) and sum the expert outputs weighted by the routing
  weights.  Permute, merge and grouping are re-orderings and copies; they do
  not change the result, which is why they are checked bit-exactly.

Readings where the sources are silent (each listed in the design notes):

* ties in routing: larger logit first, equal logits (+0 == -0) -> smaller
  expert id first; slots are stored in that order;
* non-finite logits are rejected;
* permuted rows are grouped by ascending expert id and, inside a group, kept
  in ascending assignment index a = t*k + j (a stable counting sort);
* merged-buffer slots are assigned in ascending expert id;
* bf16 workloads store the SwiGLU activation h in bf16 (round to nearest
  even) before the down projection; y_perm and y stay in wider precision;
* the multi-layer pipeline uses x_{l+1} = bf16(x_l + MoE_l(bf16(x_l W_l^T))).

Parity: every function here is pinned by ``tests/test_oracle_pins.py`` against
brute force, library routines, closed forms or invariants.
"""
from __future__ import annotations

from typing import Callable, Dict, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "round_to_bf16", "decode", "route", "expert_counts",
    "expert_offsets", "permutation", "gather_rows", "slot_map", "merge",
    "expert_matrices", "silu", "swiglu_ffn", "grouped_swiglu", "combine",
    "moe_layer", "moe_layer_tokens", "dense_standin", "residual", "pipeline",
]


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (float64 result).

    bf16 keeps 8 significant bits and fp32's exponent range.  For
    |v| in [2**(e-1), 2**e) the spacing of bf16 values is 2**(e-8); below the
    smallest normal 2**-126 the spacing is fixed at 2**-133.  ``np.rint``
    rounds half to even, and dividing by a power of two is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(v / q) * q
    big = np.abs(r) > np.float64(3.3895313892515355e38)   # above bf16 max -> inf
    return np.where(big, np.copysign(np.inf, v), r)


def decode(a: np.ndarray) -> np.ndarray:
    """Input array -> float64: uint16 is read as bf16 bits, floats are widened."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# routing, counts, permutation, gather
# ----------------------------------------------------------------------------

def route(logits: np.ndarray, k: int):
    """Top-k routing with weights renormalised over the chosen k.

    For every token t the k chosen experts are the first k of the experts
    sorted by (logit descending, expert id ascending); ``idx[t, j]`` is the
    j-th of them.  ``w[t, j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)``,
    which equals the softmax over all E experts renormalised over the chosen
    k (the full denominator cancels).  Computed in float64, stored as float32.
    """
    L = np.asarray(logits)
    if L.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError(f"k={k} out of range for E={E}")
    if not np.all(np.isfinite(L)):
        raise ValueError("non-finite router logit")
    L64 = L.astype(np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        order = np.argsort(-L64[t], kind="stable")[:k]
        chosen = L64[t, order]
        ex = np.exp(chosen - chosen[0])
        idx[t] = order
        w[t] = (ex / ex.sum()).astype(np.float32)
    return idx, w


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of (token, slot) assignments routed to expert e."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """offsets[E+1]: exclusive prefix sum of counts; offsets[E] = T*k."""
    c = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int32)


def permutation(idx: np.ndarray, E: int):
    """Stable counting sort of the assignments a = t*k + j by expert id.

    Returns ``row_of[a]`` (the row of assignment a in expert-contiguous order)
    and ``src_of[r]`` (the assignment stored in row r).  Rows of expert e are
    ``[offsets[e], offsets[e+1])`` and keep ascending a.
    """
    flat = np.asarray(idx).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    src_of = np.argsort(flat, kind="stable").astype(np.int32)
    row_of = np.empty_like(src_of)
    row_of[src_of] = np.arange(src_of.size, dtype=np.int32)
    return row_of, src_of


def gather_rows(x: np.ndarray, src_of: np.ndarray, k: int) -> np.ndarray:
    """x_perm[r] = x[src_of[r] // k] (row copy, dtype and bits preserved)."""
    return np.asarray(x)[np.asarray(src_of) // k].copy()


# ----------------------------------------------------------------------------
# merged weight buffer
# ----------------------------------------------------------------------------

def slot_map(ids: Sequence[int], E: int) -> np.ndarray:
    """slot_of[e] = position of e in the ascending id set, -1 when e is absent."""
    ids = [int(e) for e in ids]
    if sorted(set(ids)) != ids:
        raise ValueError("ids must be strictly ascending")
    s = np.full(E, -1, dtype=np.int32)
    for pos, e in enumerate(ids):
        s[e] = pos
    return s


def merge(pools: Sequence[tuple], ids: Sequence[int]) -> np.ndarray:
    """One contiguous buffer holding the blocks of ``ids`` (ascending), slot by slot.

    ``pools`` is a list of (first_id, blocks[n, elems]) pairs: pool p holds
    experts [first_id, first_id + n).  Every id must live in exactly one pool.
    The merged buffer is the contiguous weight buffer the grouped GEMM reads
    (DWDP explainer, contiguous-buffer panel).
    """
    ids = list(ids)
    if sorted(set(ids)) != ids:
        raise ValueError("ids must be strictly ascending")
    ref = pools[0][1]
    out = np.empty((len(ids), ref.shape[1]), dtype=ref.dtype)
    for pos, e in enumerate(ids):
        owners = [(f, b) for f, b in pools if f <= e < f + b.shape[0]]
        if len(owners) != 1:
            raise ValueError(f"expert {e} not in exactly one pool")
        f, b = owners[0]
        out[pos] = b[e - f]
    return out


# ----------------------------------------------------------------------------
# SwiGLU experts
# ----------------------------------------------------------------------------

def expert_matrices(block: np.ndarray, H: int, I: int, dtype=np.float64):
    """Split one expert block into (Wg [I,H], Wu [I,H], Wd [H,I]), stored out x in, as float64
    (or ``dtype``: float32 for the bulk CPU path; bf16 and fp32 values convert exactly)."""
    b = decode(block).ravel()
    if dtype != np.float64:
        b = b.astype(dtype)
    if b.size != 3 * H * I:
        raise ValueError("expert block has the wrong size")
    wg = b[: H * I].reshape(I, H)
    wu = b[H * I: 2 * H * I].reshape(I, H)
    wd = b[2 * H * I:].reshape(H, I)
    return wg, wu, wd


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x_rows: np.ndarray, wg, wu, wd, round_h: bool, dtype=np.float64) -> np.ndarray:
    """SwiGLU FFN of one expert on rows x[n, H]: (silu(x Wg^T) * (x Wu^T)) Wd^T.

    With ``round_h`` the activation h is stored as bf16 (round to nearest
    even) before the down projection, as a bf16 workload stores it.
    ``dtype`` is the arithmetic type: float64 (the definition), or float32
    for the bulk CPU path (the same steps with float32 matrix products).
    """
    x = decode(x_rows).astype(dtype)
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    if round_h:
        h = round_to_bf16(h)
    return (h.astype(dtype) @ wd.T).astype(dtype)


def grouped_swiglu(x_perm: np.ndarray, offsets: np.ndarray,
                   weights_of: Callable[[int], np.ndarray], H: int, I: int,
                   round_h: bool, dtype=np.float64) -> np.ndarray:
    """y_perm[r] = FFN_e(x_perm[r]) for the rows r of every expert group e (float64, or
    ``dtype``), one expert's weights decoded at a time."""
    xp = decode(x_perm)
    R = xp.shape[0]
    y = np.zeros((R, H), dtype=dtype)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wg, wu, wd = expert_matrices(weights_of(e), H, I, dtype)
        y[lo:hi] = swiglu_ffn(xp[lo:hi], wg, wu, wd, round_h, dtype)
    return y


def combine(y_perm: np.ndarray, row_of: np.ndarray, w: np.ndarray, k: int,
            dtype=np.float64) -> np.ndarray:
    """y[t] = sum_{j=0..k-1} w[t,j] * y_perm[row_of[t*k + j]], summed in j order (float64, or
    ``dtype``)."""
    yp = np.asarray(y_perm, dtype=dtype)
    w = np.asarray(w, dtype=dtype)
    T = w.shape[0]
    y = np.zeros((T, yp.shape[1]), dtype=dtype)
    for j in range(k):
        y += w[:, j:j + 1] * yp[np.asarray(row_of)[np.arange(T) * k + j]]
    return y


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def moe_layer(x: np.ndarray, logits: np.ndarray, k: int,
              weights_of: Callable[[int], np.ndarray], H: int, I: int,
              round_h: bool, dtype=np.float64) -> Dict[str, np.ndarray]:
    """Route -> counts/offsets -> permutation -> gather -> grouped SwiGLU -> combine.

    ``dtype`` float32 gives the bulk CPU path: the same steps, with the expert
    products and the combine in float32 (routing and permutation are exact)."""
    T, E = np.asarray(logits).shape
    idx, w = route(logits, k)
    counts = expert_counts(idx, E)
    offsets = expert_offsets(counts)
    row_of, src_of = permutation(idx, E)
    x_perm = gather_rows(x, src_of, k)
    y_perm = grouped_swiglu(x_perm, offsets, weights_of, H, I, round_h, dtype)
    y = combine(y_perm, row_of, w, k, dtype)
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, row_of=row_of,
                src_of=src_of, x_perm=x_perm, y_perm=y_perm, y=y)


def moe_layer_tokens(x: np.ndarray, logits: np.ndarray, k: int,
                     weights_of: Callable[[int], np.ndarray], H: int, I: int,
                     round_h: bool, tokens: Sequence[int]) -> Dict[str, np.ndarray]:
    """The layer output for selected tokens only, straight from the definition.

    y[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t]), with no permutation or merge
    involved; each needed expert is decoded once.  Used for sampled checks at
    sizes where the whole layer is too slow on the CPU.
    """
    tokens = [int(t) for t in tokens]
    L = np.asarray(logits)[tokens]
    idx, w = route(L, k)
    xs = decode(np.asarray(x)[tokens])
    need: Dict[int, list] = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            need.setdefault(int(idx[i, j]), []).append((i, j))
    contrib = np.zeros((len(tokens), k, H), dtype=np.float64)
    for e in sorted(need):
        wg, wu, wd = expert_matrices(weights_of(e), H, I)
        rows = [i for i, _ in need[e]]
        out = swiglu_ffn(xs[rows], wg, wu, wd, round_h)
        for (i, j), o in zip(need[e], out):
            contrib[i, j] = o
    y = np.zeros((len(tokens), H), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1].astype(np.float64) * contrib[:, j]
    return dict(idx=idx, w=w, y=y, expert_out=contrib)


# ----------------------------------------------------------------------------
# multi-layer pipeline with the dense stand-in block
# ----------------------------------------------------------------------------

def dense_standin(x: np.ndarray, w_attn: np.ndarray) -> np.ndarray:
    """A = bf16(x W^T): the dense block that stands in for attention (float64 result on the bf16 grid)."""
    return round_to_bf16(decode(x) @ decode(w_attn).T)


def residual(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """x_next = bf16(x + y) (float64 result on the bf16 grid)."""
    return round_to_bf16(decode(x) + np.asarray(y, dtype=np.float64))


def pipeline(x0: np.ndarray, layers: Sequence[dict], k: int, H: int, I: int) -> list:
    """Run the layers in order: A_l = dense(x_l); y_l = MoE_l(A_l); x_{l+1} = bf16(x_l + y_l).

    ``layers[l]`` holds ``logits``, ``w_attn`` and ``weights_of``.  Returns the
    list of per-layer dicts with ``x_in``, ``a``, ``y`` and ``x_out`` (float64).
    """
    out = []
    x = decode(x0)
    for spec in layers:
        a = dense_standin(x, spec["w_attn"])
        res = moe_layer(a, spec["logits"], k, spec["weights_of"], H, I, round_h=True)
        x_next = residual(x, res["y"])
        out.append(dict(x_in=x, a=a, y=res["y"], x_out=x_next, layer=res))
        x = x_next
    return out
