"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random inputs and packs them into the byte layouts the
library consumes.  It holds none of the layer's arithmetic (no routing, no
permutation, no GEMM, no combine), so both the HIP path and the CPU oracle can
take their inputs from it without sharing any of the method.

Workloads.  The pages (DWDP, arXiv 2604.01621v1, abstract; DWDP explainer,
"weight-level imbalance" panel) evaluate DeepSeek-R1 serving; neither trained
weights nor traces are available here, so every tensor is a seeded Gaussian
stand-in with the R1 MoE shape (256 routed experts, hidden 7168, SwiGLU
intermediate 2048, top-8), or the tiny fp32 layer used for exact checks.

Expert block layout (one expert, row-major, ``dtype`` elements)::

    [ Wg : I rows x H cols ][ Wu : I rows x H cols ][ Wd : H rows x I cols ]

i.e. every matrix is stored output-major ("out x in"), so ``g = x @ Wg.T``.
The reduction dimension is contiguous in memory for both GEMMs.

Seeds: every draw comes from ``numpy.random.default_rng([seed, layer, stream,
...])`` (PCG64 seeded through a SeedSequence) on the host, or, for the
multi-GB R1 weight pools, from a ``torch.Generator`` seeded per expert on the
device that will hold the pool.  Either way the oracle reads back the very
bytes the GPU consumes, so no cross-platform generator agreement is needed.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "config", "logits", "activations", "to_bf16_bits",
    "expert_block_elems", "expert_block_bytes", "expert_block_np", "pool_np",
    "pool_torch", "dense_weight_np", "dense_weight_torch", "digest",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens in the batch
    H: int            # hidden size
    I: int            # SwiGLU intermediate size per expert
    E: int            # routed experts
    k: int            # experts chosen per token
    dtype: str        # "f32" or "bf16": dtype of x and of the expert weights
    n_local: int      # experts [0, n_local) are this rank's share; the rest are remote
    layers: int = 1
    zipf_s: Optional[float] = None   # per-expert Zipf bias on the logits
    seed: int = 0
    rho_seed: Optional[int] = None   # seed of the hot-expert ranking for the Zipf bias
    dense_standin: bool = False      # a dense H x H GEMM per layer before the MoE block

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


_R1 = dict(H=7168, I=2048, E=256, k=8, dtype="bf16", n_local=64)

CONFIGS = {
    # tiny exact-check layer: experts 0-3 local, 4-7 in the remote pool
    "tiny_fp32_t64": MoEConfig("tiny_fp32_t64", T=64, H=256, I=512, E=8, k=2,
                               dtype="f32", n_local=4, seed=101),
    # DeepSeek-R1-shaped decode step, 4-rank group: 64 local, 192 remote
    "r1_decode_t64": MoEConfig("r1_decode_t64", T=64, seed=202, **_R1),
    # R1-shaped prefill with Zipf(1.1) expert skew (weight-level imbalance)
    "r1_prefill_t8192_zipf": MoEConfig("r1_prefill_t8192_zipf", T=8192, seed=303,
                                       zipf_s=1.1, rho_seed=304, **_R1),
    # R1-shaped layer at 16384 tokens, uniform routing
    "r1_prefill_t16384": MoEConfig("r1_prefill_t16384", T=16384, seed=404, **_R1),
    # 6-layer pipeline, 4096 tokens per layer, dense stand-in block per layer
    "r1_pipeline_6x4096": MoEConfig("r1_pipeline_6x4096", T=4096, seed=505, layers=6,
                                    dense_standin=True, **_R1),
    # 4-layer pipeline at 16384 tokens per layer: compute per layer well above the prefetch
    "r1_pipeline_4x16384": MoEConfig("r1_pipeline_4x16384", T=16384, seed=606, layers=4,
                                     dense_standin=True, **_R1),
}
# DWDP3: a 3-rank group holds 86 of the 256 experts locally and fetches 170
_R1_3 = dict(_R1, n_local=86)
CONFIGS["r1_decode_t64_dwdp3"] = MoEConfig("r1_decode_t64_dwdp3", T=64, seed=202, **_R1_3)
CONFIGS["r1_pipeline_6x4096_dwdp3"] = MoEConfig("r1_pipeline_6x4096_dwdp3", T=4096, seed=505,
                                                 layers=6, dense_standin=True, **_R1_3)


def config(name: str) -> MoEConfig:
    return CONFIGS[name]


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.default_rng([int(v) for v in entropy])


def logits(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Router logits f32[T, E] ~ N(0, 1), plus a Zipf(s) bias per expert when set.

    The bias of expert e is ``-s * ln(rho(e))`` with rho a seeded permutation
    of 1..E, so the softmax mass of expert e scales like rho(e)**-s and the hot
    experts are spread over the local and the remote id ranges.
    """
    z = _rng(cfg.seed, layer, 0).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.zipf_s is not None:
        rho = _rng(cfg.rho_seed if cfg.rho_seed is not None else cfg.seed + 1).permutation(cfg.E) + 1
        bias = (-cfg.zipf_s * np.log(rho.astype(np.float64))).astype(np.float32)
        z = (z + bias[None, :]).astype(np.float32)
    return np.ascontiguousarray(z)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Layer input x[T, H] ~ N(0, 1): float32 for f32 configs, bf16 bits (uint16) otherwise."""
    x = _rng(cfg.seed, layer, 1).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return x if cfg.dtype == "f32" else to_bf16_bits(x)


def expert_block_elems(cfg: MoEConfig) -> int:
    return 3 * cfg.H * cfg.I


def expert_block_bytes(cfg: MoEConfig) -> int:
    return expert_block_elems(cfg) * cfg.elem_bytes


def expert_block_np(cfg: MoEConfig, layer: int, e: int) -> np.ndarray:
    """One expert block drawn on the host: Wg, Wu ~ N(0, std 1/sqrt(H)), Wd ~ N(0, std 1/sqrt(I)).

    Returns float32[3*H*I] for f32 configs, bf16 bits uint16[3*H*I] otherwise.
    """
    g = _rng(cfg.seed, layer, 2, e)
    H, I = cfg.H, cfg.I
    blk = np.empty(3 * H * I, dtype=np.float32)
    blk[: 2 * H * I] = g.standard_normal(2 * H * I, dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
    blk[2 * H * I:] = g.standard_normal(H * I, dtype=np.float32) * np.float32(1.0 / math.sqrt(I))
    return blk if cfg.dtype == "f32" else to_bf16_bits(blk)


def pool_np(cfg: MoEConfig, layer: int, ids: Sequence[int]) -> np.ndarray:
    """Contiguous host pool [len(ids), 3*H*I] of the given experts (small shapes only)."""
    ids = list(ids)
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    out = np.empty((len(ids), expert_block_elems(cfg)), dtype=dt)
    for i, e in enumerate(ids):
        out[i] = expert_block_np(cfg, layer, e)
    return out


def _torch_seed(cfg: MoEConfig, layer: int, stream: int, e: int) -> int:
    h = hashlib.sha256(f"{cfg.seed}/{layer}/{stream}/{e}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def pool_torch(cfg: MoEConfig, layer: int, first: int, n: int, device, out=None):
    """Contiguous pool of experts [first, first+n) drawn with torch on ``device``.

    Returns a torch tensor [n, 3*H*I] (float32 or bfloat16).  Each expert has
    its own generator seed, so any subset can be regenerated independently.
    ``out`` may be a preallocated tensor of that shape and dtype.
    """
    import torch
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    H, I = cfg.H, cfg.I
    if out is None:
        out = torch.empty((n, 3 * H * I), dtype=tdt, device=device)
    gen = torch.Generator(device=device)
    buf = torch.empty(H * I, dtype=torch.float32, device=device)
    for i in range(n):
        e = first + i
        gen.manual_seed(_torch_seed(cfg, layer, 2, e))
        for m in range(3):
            torch.randn(H * I, generator=gen, out=buf)
            buf.mul_(1.0 / math.sqrt(H if m < 2 else I))
            out[i, m * H * I:(m + 1) * H * I].copy_(buf)
    return out


def dense_weight_np(cfg: MoEConfig, layer: int) -> np.ndarray:
    """Dense stand-in weight W[H, H] (out x in) ~ N(0, std 1/sqrt(H)), host, small shapes."""
    w = _rng(cfg.seed, layer, 3).standard_normal((cfg.H, cfg.H), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(cfg.H))
    return w if cfg.dtype == "f32" else to_bf16_bits(w)


def dense_weight_torch(cfg: MoEConfig, layer: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(cfg, layer, 3, 0))
    w = torch.randn((cfg.H, cfg.H), generator=gen, device=device, dtype=torch.float32)
    w.mul_(1.0 / math.sqrt(cfg.H))
    return w.to(torch.float32 if cfg.dtype == "f32" else torch.bfloat16)


def digest(a) -> str:
    """SHA-256 of an array's bytes (numpy or torch), for recording input identity."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().view(-1).view(__import__("torch").uint8).numpy()
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
