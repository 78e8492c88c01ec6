"""The library's host code (argument validation, workspace layout, launch
planning) under AddressSanitizer and UBSan, on the CPU: every HIP source is
compiled with the sanitizers on its host pass only (the GPU code is built as
usual), linked into a separate library, and driven by tests/host_abi_checks.cpp
through every validation path of the C ABI.  No GPU is needed: each call is
rejected before anything is enqueued, or only sizes a workspace."""
import concurrent.futures
import os
import subprocess

import pytest

from spatial_sparse_attention_ssa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stderr[-4000:]}")
    return res


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([_build.hipcc(), *flags, *SAN, f"-I{_build.INCLUDE}", f"-I{_build.CSRC}", "-c", src, "-o", obj])
    return obj


@pytest.fixture(scope="module")
def sanitized_driver():
    try:
        hipcc = _build.hipcc()
    except RuntimeError:
        pytest.skip("no ROCm toolchain")
    os.makedirs(OUT, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, _build.sources()))
    lib = os.path.join(OUT, "libssa_san.so")
    _run([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    exe = os.path.join(OUT, "host_abi_checks")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    _run([clang, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          f"-I{_build.INCLUDE}", os.path.join(ROOT, "tests", "host_abi_checks.cpp"), lib,
          f"-Wl,-rpath,{OUT}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def test_host_code_clean_under_asan_and_ubsan(sanitized_driver):
    env = dict(os.environ)
    # the HIP runtime keeps its own allocations until exit: leak reports off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " 0 failed" in res.stdout
