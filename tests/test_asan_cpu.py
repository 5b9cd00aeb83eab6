"""The library's host code (argument checks, id and pool checks, copy planning, error text)
under AddressSanitizer, on the CPU: libmoe.so rebuilt with the sanitizer on its host side
only (the GPU code is built as usual), and the plain C99 caller of the C ABI built with the
sanitizer, linked against it and run.  No GPU is touched: every entry point the caller uses
answers on the host."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_gemm_weights_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
LLVM = "/opt/rocm/llvm/bin"
# the sanitizer instruments host code only: -Xarch_host before each host-side flag
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime_dir():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(hits[0]) if hits else None


@pytest.fixture(scope="module")
def asan_build(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(os.path.join(LLVM, "clang++")):
        pytest.skip("ROCm compilers not found")
    rt = _asan_runtime_dir()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime")
    out = str(tmp_path_factory.mktemp("asan"))

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
               "-I", INCLUDE, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    lib = os.path.join(out, "libmoe_asan.so")
    r = subprocess.run([os.path.join(LLVM, "clang++"), "-shared", "-fPIC", "-fsanitize=address",
                        "-shared-libasan", "-o", lib, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = os.path.join(out, "c_abi_consumer_asan")
    r = subprocess.run([os.path.join(LLVM, "clang"), "-std=c99", "-Wall", "-Wextra", "-pedantic",
                        "-Werror", "-g", "-fsanitize=address", "-shared-libasan", "-I", INCLUDE,
                        os.path.join(ROOT, "tests", "c_abi_consumer.c"), "-o", exe, "-L", out,
                        "-lmoe_asan", f"-Wl,-rpath,{out}", f"-Wl,-rpath,{rt}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe, lib


def _run(exe, extra_env=None):
    env = dict(os.environ)
    # leaks of the HIP runtime at exit are not this library's; every other error is fatal
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env.update(extra_env or {})
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_library_host_code_is_instrumented(asan_build):
    _, lib = asan_build
    nm = shutil.which("nm") or os.path.join(LLVM, "llvm-nm")
    syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_load" in syms


def test_c_caller_under_address_sanitizer(asan_build):
    r = _run(asan_build[0])
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert r.stdout.startswith("ok moe-gfx950")


def test_c_caller_under_address_sanitizer_debug_sync(asan_build):
    """The debug mode's checks run only after a call has enqueued work, so the argument
    errors are unchanged with it on."""
    r = _run(asan_build[0], {"MOE_DEBUG_SYNC": "1"})
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
