"""The host front end (hyb_api.cpp: argument checks, workspace sizing, error strings) built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code, then driven through every C-ABI
host check of test_abi.py in a process with the sanitizer runtime preloaded. The device code and
the other sources are the normal build's objects. Needs no GPU."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from sparse_attention_hyb_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# each sanitizer flag applies to the host pass only (the device code is not instrumented)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_front_end_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "hyb_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run the build first)")
    api_obj = str(tmp_path / "hyb_api_san.o")
    cmd = [hipcc, "-x", "hip"] + B.FLAGS + HOST_SAN + ["-g", "-c", os.path.join(B.CSRC, "hyb_api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    lib = str(tmp_path / "libhyb_san.so")
    cmd = [hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC"] + HOST_SAN + ["-o", lib, api_obj] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    nm = shutil.which("nm")
    if nm:   # the host code is instrumented: it calls the sanitizers' report hooks
        syms = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt[-1]
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_abi.py"), lib],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
