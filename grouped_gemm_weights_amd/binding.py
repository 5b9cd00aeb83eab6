"""ctypes binding of ``libmoe.so`` (include/moe.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does
nothing but convert arguments (torch tensors -> device pointers, torch streams
-> hipStream_t) and turn a negative return code into ``MoEError``.  All the
work runs in the HIP kernels of the library.  There is no fallback: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_STATUS = -5
MOE_STATUS_NONFINITE_LOGIT, MOE_STATUS_EXPERT_ABSENT, MOE_STATUS_BAD_EXPERT_ID = 1, 2, 4
MOE_COPY_SDMA, MOE_COPY_ANY, MOE_COPY_KERNEL = 0, 1, 2


def copy_kernel_on(n_blocks: int) -> int:
    """MOE_COPY_KERNEL_ON(n): the library's copy kernel on at most n workgroups (0: no limit)."""
    if not 0 <= n_blocks <= 0xFFFF:
        raise ValueError(f"copy kernel workgroups {n_blocks} outside [0, 65535]")
    return MOE_COPY_KERNEL | (n_blocks << 8)

# Every symbol include/moe.h declares (checked by the CPU tests).
EXPORTS = (
    "moe_route", "moe_permute_workspace_size", "moe_permute", "moe_permute_noalloc",
    "moe_merge_weights",
    "moe_prefetch_layer", "moe_prefetch_routed", "moe_grouped_swiglu_workspace_size",
    "moe_grouped_swiglu",
    "moe_grouped_swiglu_range", "moe_grouped_swiglu_gathered", "moe_grouped_swiglu_combine",
    "moe_combine", "moe_dense_gemm", "moe_residual_add", "moe_event_create",
    "moe_event_destroy", "moe_event_record", "moe_event_elapsed_ms", "moe_stream_wait_event",
    "moe_last_error", "moe_version", "moe_vmm_granularity", "moe_vmm_create", "moe_vmm_map",
    "moe_vmm_unmap", "moe_vmm_release",
)


class MoEError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed ({code}): {text}")
        self.code = code


class MoePool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("expert_bytes", ctypes.c_int64),
                ("first_expert", ctypes.c_int32), ("n_experts", ctypes.c_int32)]


class MoeWbuf(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("expert_bytes", ctypes.c_int64),
                ("n_slots", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("slot_of", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m grouped_gemm_weights_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "moe_route": [P, I, I, I, P, P, P, P],
        "moe_permute_workspace_size": [I, I, I, PSZ],
        "moe_permute": [P, I, I, I, P, I, I, P, P, P, P, P, P, SZ, P, P],
        "moe_permute_noalloc": [P, I, I, I, P, I, I, P, P, P, P, P, P, P],
        "moe_merge_weights": [ctypes.POINTER(MoePool), P, I, ctypes.POINTER(MoeWbuf), P, P, P, I],
        "moe_prefetch_layer": [ctypes.POINTER(MoePool), P, I, ctypes.POINTER(MoeWbuf), P, P, P, I],
        "moe_prefetch_routed": [ctypes.POINTER(MoePool), P, ctypes.POINTER(MoeWbuf), P, P, P, P, I],
        "moe_grouped_swiglu_workspace_size": [I, I, I, I, I, PSZ],
        "moe_grouped_swiglu": [P, P, I, I, I, I, I, ctypes.POINTER(MoeWbuf), P, SZ, P, P, P],
        "moe_grouped_swiglu_range": [P, P, I, I, I, I, I, ctypes.POINTER(MoeWbuf), I, I, P, SZ, P, P, P],
        "moe_grouped_swiglu_gathered": [P, P, I, P, I, I, I, I, I, ctypes.POINTER(MoeWbuf), I, I, P, SZ,
                                        P, P, P],
        "moe_grouped_swiglu_combine": [P, P, P, I, I, P, I, I, I, I, ctypes.POINTER(MoeWbuf), P, SZ,
                                       P, P, P],
        "moe_combine": [P, P, P, I, I, I, P, P],
        "moe_dense_gemm": [P, P, I, I, I, P, P],
        "moe_residual_add": [P, P, I64, P, P],
        "moe_event_create": [ctypes.POINTER(ctypes.c_void_p), I],
        "moe_event_destroy": [P],
        "moe_event_record": [P, P],
        "moe_event_elapsed_ms": [P, P, ctypes.POINTER(ctypes.c_float)],
        "moe_stream_wait_event": [P, P],
        "moe_vmm_granularity": [I, PSZ],
        "moe_vmm_create": [I, SZ, ctypes.POINTER(ctypes.c_void_p)],
        "moe_vmm_map": [I, ctypes.POINTER(ctypes.c_void_p), PSZ, I, ctypes.POINTER(ctypes.c_void_p)],
        "moe_vmm_unmap": [P, PSZ, I],
        "moe_vmm_release": [P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoEError(fn, rc, lib.moe_last_error().decode())


def ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(s) -> Optional[int]:
    """hipStream_t of a torch stream (or an int handle; None = the null stream)."""
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _ids_arg(ids: Sequence[int]):
    arr = (ctypes.c_int32 * len(ids))(*[int(e) for e in ids])
    return arr, len(ids)


def pool(base, expert_bytes: int, first_expert: int, n_experts: int) -> MoePool:
    return MoePool(ptr(base), int(expert_bytes), int(first_expert), int(n_experts))


def wbuf(base, expert_bytes: int, n_slots: int, n_experts: int, slot_of) -> MoeWbuf:
    return MoeWbuf(ptr(base), int(expert_bytes), int(n_slots), int(n_experts), ptr(slot_of))


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def moe_route(logits, T, E, k, topk_idx, topk_w, status=None, stream=None):
    _check("moe_route", lib.moe_route(ptr(logits), T, E, k, ptr(topk_idx), ptr(topk_w),
                                      ptr(status), stream_handle(stream)))


def moe_permute_workspace_size(T, E, k) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_permute_workspace_size", lib.moe_permute_workspace_size(T, E, k, ctypes.byref(n)))
    return n.value


def moe_permute(topk_idx, T, E, k, x, H, dtype, counts, offsets, row_of, src_of, x_perm,
                ws, ws_bytes, status=None, stream=None):
    _check("moe_permute", lib.moe_permute(ptr(topk_idx), T, E, k, ptr(x), H, dtype, ptr(counts),
                                          ptr(offsets), ptr(row_of), ptr(src_of), ptr(x_perm),
                                          ptr(ws), ws_bytes, ptr(status), stream_handle(stream)))


def moe_permute_noalloc(topk_idx, T, E, k, x, H, dtype, counts, offsets, row_of, src_of, x_perm,
                        status=None, stream=None):
    _check("moe_permute_noalloc",
           lib.moe_permute_noalloc(ptr(topk_idx), T, E, k, ptr(x), H, dtype, ptr(counts),
                                   ptr(offsets), ptr(row_of), ptr(src_of), ptr(x_perm),
                                   ptr(status), stream_handle(stream)))


def moe_merge_weights(local: MoePool, ids: Sequence[int], dst: MoeWbuf, stream=None,
                      wait_free=None, ready=None, copy_mode=MOE_COPY_SDMA):
    arr, n = _ids_arg(ids)
    _check("moe_merge_weights", lib.moe_merge_weights(ctypes.byref(local), arr, n, ctypes.byref(dst),
                                                      stream_handle(stream), wait_free, ready,
                                                      copy_mode))


def moe_prefetch_layer(remote: MoePool, ids: Sequence[int], dst: MoeWbuf, copy_stream=None,
                       wait_free=None, ready=None, copy_mode=MOE_COPY_SDMA):
    arr, n = _ids_arg(ids)
    _check("moe_prefetch_layer", lib.moe_prefetch_layer(ctypes.byref(remote), arr, n,
                                                        ctypes.byref(dst),
                                                        stream_handle(copy_stream), wait_free,
                                                        ready, copy_mode))


def moe_prefetch_routed(remote: MoePool, counts, dst: MoeWbuf, copy_stream=None,
                        counts_ready=None, wait_free=None, ready=None, max_blocks: int = 0):
    _check("moe_prefetch_routed", lib.moe_prefetch_routed(ctypes.byref(remote), ptr(counts),
                                                          ctypes.byref(dst),
                                                          stream_handle(copy_stream), counts_ready,
                                                          wait_free, ready, max_blocks))


def moe_grouped_swiglu_workspace_size(R, E, H, I, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_grouped_swiglu_workspace_size",
           lib.moe_grouped_swiglu_workspace_size(R, E, H, I, dtype, ctypes.byref(n)))
    return n.value


def moe_grouped_swiglu(x_perm, offsets, R, E, H, I, dtype, w: MoeWbuf, ws, ws_bytes, y_perm,
                       status=None, stream=None):
    _check("moe_grouped_swiglu", lib.moe_grouped_swiglu(ptr(x_perm), ptr(offsets), R, E, H, I, dtype,
                                                        ctypes.byref(w), ptr(ws), ws_bytes,
                                                        ptr(y_perm), ptr(status),
                                                        stream_handle(stream)))


def moe_grouped_swiglu_range(x_perm, offsets, R, E, H, I, dtype, w: MoeWbuf, e_begin, e_end, ws,
                             ws_bytes, y_perm, status=None, stream=None):
    _check("moe_grouped_swiglu_range",
           lib.moe_grouped_swiglu_range(ptr(x_perm), ptr(offsets), R, E, H, I, dtype, ctypes.byref(w),
                                        e_begin, e_end, ptr(ws), ws_bytes, ptr(y_perm), ptr(status),
                                        stream_handle(stream)))


def moe_grouped_swiglu_gathered(x, src_of, k, offsets, R, E, H, I, dtype, w: MoeWbuf, e_begin, e_end,
                                ws, ws_bytes, y_perm, status=None, stream=None):
    _check("moe_grouped_swiglu_gathered",
           lib.moe_grouped_swiglu_gathered(ptr(x), ptr(src_of), k, ptr(offsets), R, E, H, I, dtype,
                                           ctypes.byref(w), e_begin, e_end, ptr(ws), ws_bytes,
                                           ptr(y_perm), ptr(status), stream_handle(stream)))


def moe_grouped_swiglu_combine(x, src_of, topk_w, T, k, offsets, E, H, I, dtype, w: MoeWbuf, ws,
                               ws_bytes, y, status=None, stream=None):
    _check("moe_grouped_swiglu_combine",
           lib.moe_grouped_swiglu_combine(ptr(x), ptr(src_of), ptr(topk_w), T, k, ptr(offsets), E, H,
                                          I, dtype, ctypes.byref(w), ptr(ws), ws_bytes, ptr(y),
                                          ptr(status), stream_handle(stream)))


def moe_combine(y_perm, row_of, topk_w, T, k, H, y, stream=None):
    _check("moe_combine", lib.moe_combine(ptr(y_perm), ptr(row_of), ptr(topk_w), T, k, H, ptr(y),
                                          stream_handle(stream)))


def moe_dense_gemm(x, w, M, N, K, out, stream=None):
    _check("moe_dense_gemm", lib.moe_dense_gemm(ptr(x), ptr(w), M, N, K, ptr(out),
                                                stream_handle(stream)))


def moe_residual_add(x, y, n, out, stream=None):
    _check("moe_residual_add", lib.moe_residual_add(ptr(x), ptr(y), n, ptr(out),
                                                    stream_handle(stream)))


def moe_event_create(timing: bool = False) -> int:
    ev = ctypes.c_void_p(0)
    _check("moe_event_create", lib.moe_event_create(ctypes.byref(ev), 1 if timing else 0))
    return ev.value


def moe_event_destroy(ev) -> None:
    _check("moe_event_destroy", lib.moe_event_destroy(ev))


def moe_event_record(ev, stream=None) -> None:
    _check("moe_event_record", lib.moe_event_record(ev, stream_handle(stream)))


def moe_event_elapsed_ms(start, stop) -> float:
    ms = ctypes.c_float(0.0)
    _check("moe_event_elapsed_ms", lib.moe_event_elapsed_ms(start, stop, ctypes.byref(ms)))
    return ms.value


def moe_stream_wait_event(stream, ev) -> None:
    _check("moe_stream_wait_event", lib.moe_stream_wait_event(stream_handle(stream), ev))


def moe_vmm_granularity(device: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_vmm_granularity", lib.moe_vmm_granularity(device, ctypes.byref(n)))
    return n.value


def moe_vmm_create(nbytes: int, device: int = 0) -> int:
    h = ctypes.c_void_p(0)
    _check("moe_vmm_create", lib.moe_vmm_create(device, nbytes, ctypes.byref(h)))
    return h.value


def moe_vmm_map(phys: Sequence[int], sizes: Sequence[int], device: int = 0) -> int:
    n = len(phys)
    ph = (ctypes.c_void_p * n)(*phys)
    sz = (ctypes.c_size_t * n)(*sizes)
    va = ctypes.c_void_p(0)
    _check("moe_vmm_map", lib.moe_vmm_map(device, ph, sz, n, ctypes.byref(va)))
    return va.value


def moe_vmm_unmap(va: int, sizes: Sequence[int]) -> None:
    n = len(sizes)
    sz = (ctypes.c_size_t * n)(*sizes)
    _check("moe_vmm_unmap", lib.moe_vmm_unmap(va, sz, n))


def moe_vmm_release(phys: int) -> None:
    _check("moe_vmm_release", lib.moe_vmm_release(phys))


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def moe_version() -> str:
    return lib.moe_version().decode()
