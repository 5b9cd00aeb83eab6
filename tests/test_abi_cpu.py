"""The C-ABI library loads and exports every symbol include/moe.h declares,
and rejects bad arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "grouped_gemm_weights_amd", "libmoe.so")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def B():
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built (run `python -m grouped_gemm_weights_amd.build`)")
    from grouped_gemm_weights_amd import binding
    return binding


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ["moe_route", "moe_permute", "moe_merge_weights", "moe_grouped_swiglu",
                     "moe_combine", "moe_prefetch_layer"]:
        assert required in names


def test_library_exports_every_header_symbol(B):
    lib = ctypes.CDLL(LIB)
    for name in header_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert sorted(B.EXPORTS) == header_functions()
    assert B.moe_version().startswith("moe-gfx950")


def test_host_side_argument_errors(B):
    with pytest.raises(B.MoEError) as e:
        B.moe_route(0, 4, 8, 9, 0, 0)                     # k > E
    assert e.value.code == B.MOE_ERR_ARG
    with pytest.raises(B.MoEError) as e:
        B.moe_route(0, 4, 2048, 2, 0, 0)                  # E above the kernel limit
    assert e.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoEError) as e:
        B.moe_permute(1, 4, 8, 2, 1, 16, B.MOE_BF16, 1, 1, 1, 1, None, 0, 0)   # no workspace
    assert e.value.code == B.MOE_ERR_WORKSPACE
    buf = B.wbuf(1 << 20, 96, 4, 8, 1 << 21)
    pool = B.pool(1 << 22, 96, 0, 4)
    for ids in ([3, 1], [0, 8], [0, 1, 2, 3, 4]):      # unsorted, out of range, too many
        with pytest.raises(B.MoEError) as e:
            B.moe_merge_weights(pool, ids, buf)
        assert e.value.code == B.MOE_ERR_ARG
    with pytest.raises(B.MoEError) as e:
        B.moe_prefetch_layer(B.pool(1 << 22, 64, 4, 4), [4], buf)   # block size mismatch
    assert e.value.code == B.MOE_ERR_ARG
    # copy modes: unknown kind, a workgroup count on a runtime copy kind, negative
    for mode in (3, B.MOE_COPY_ANY | (4 << 8), B.MOE_COPY_SDMA | (1 << 8), -1):
        with pytest.raises(B.MoEError) as e:
            B.moe_prefetch_layer(B.pool(1 << 22, 96, 4, 4), [4], buf, copy_mode=mode)
        assert e.value.code == B.MOE_ERR_ARG
    assert B.copy_kernel_on(32) == (2 | 32 << 8)
    with pytest.raises(ValueError):
        B.copy_kernel_on(1 << 16)
    with pytest.raises(B.MoEError) as e:
        B.moe_grouped_swiglu(1, 1, 8, 8, 1 << 16, 1 << 15, B.MOE_BF16,
                             B.wbuf(1, 3 * (1 << 31) * 2, 8, 8, 1), 1, 1 << 40, 1)
    assert e.value.code == B.MOE_ERR_UNSUPPORTED                  # H*I = 2^31
    with pytest.raises(B.MoEError) as e:
        B.moe_grouped_swiglu(1, 1, 8, 8, 12, 8, B.MOE_BF16, B.wbuf(1, 3 * 12 * 8 * 2, 8, 8, 1), 1, 1 << 30, 1)
    assert e.value.code == B.MOE_ERR_UNSUPPORTED                  # H not a multiple of 8
    with pytest.raises(B.MoEError) as e:
        B.moe_grouped_swiglu(1, 1, 8, 8, 16, 8, B.MOE_BF16, B.wbuf(1, 3 * 16 * 8 * 2, 8, 8, 1), 1, 16, 1)
    assert e.value.code == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoEError) as e:
        B.moe_combine(1, 1, 1, 4, 65, 8, 1)                       # k above the limit
    assert e.value.code == B.MOE_ERR_UNSUPPORTED
    assert "moe_combine" in B.moe_last_error()


def test_workspace_sizes(B):
    assert B.moe_permute_workspace_size(0, 8, 2) == 0
    assert B.moe_permute_workspace_size(16384, 256, 8) >= 2 * 256 * 256 * 4
    R, I = 65536, 2048
    assert B.moe_grouped_swiglu_workspace_size(R, 256, 7168, I, B.MOE_BF16) >= R * I * 2


def test_plain_c_caller(B, tmp_path):
    """include/moe.h compiles as C99 with -Wall -Wextra -pedantic -Werror, a C program links
    against libmoe.so, and its host-only entry points answer (tests/c_abi_consumer.c)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_abi_consumer")
    libdir = os.path.dirname(LIB)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_consumer.c"),
           "-o", exe, "-L", libdir, "-lmoe", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok moe-gfx950")


def test_injected_prefetch_fault(B, monkeypatch):
    """MOE_INJECT_FAULT=prefetch makes moe_prefetch_layer fail as a failed HIP call would,
    before any argument is looked at (so no device memory is needed here); other sites and an
    unset variable leave it alone."""
    lib = ctypes.CDLL(LIB)
    lib.moe_last_error.restype = ctypes.c_char_p
    call = lambda: lib.moe_prefetch_layer(None, None, 0, None, None, None, None, 0)
    monkeypatch.setenv("MOE_INJECT_FAULT", "prefetch")
    assert call() == B.MOE_ERR_HIP
    assert b"fault injected" in lib.moe_last_error()
    monkeypatch.setenv("MOE_INJECT_FAULT", "merge")
    assert call() == B.MOE_ERR_ARG                     # the real argument check runs again
    monkeypatch.delenv("MOE_INJECT_FAULT")
    assert call() == B.MOE_ERR_ARG
