"""Host sanitizers: libaqlm_mi355x with AddressSanitizer and UndefinedBehaviorSanitizer
on its host code (hipcc -Xarch_host -fsanitize=...; device code unchanged), the
host-core kernel and the oracle built the same way, driven by tests/sanitize_check.c:
argument validation, the kernel-choice and workspace logic over many shapes, and the
CPU kernel against the oracle.  No GPU is used; the sanitizers abort the run on a
finding (leak detection is off: the HIP runtime keeps allocations until exit)."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd[:3])} ... failed:\n{r.stdout}\n{r.stderr[-4000:]}")
    return r


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") and os.path.exists(f"{LLVM}/clang")),
                    reason="needs the ROCm toolchain")
def test_host_code_under_asan_ubsan(tmp_path):
    from additive_quantized_gemv_amd import build as b
    csrc, inc = b.CSRC, b.INCLUDE
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]

    def hip_obj(src):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([b.HIPCC, *b.FLAGS, "-O1", *host_san, *lang, "-c", os.path.join(csrc, src), "-o", obj])
        return obj

    def cpu_obj():
        obj = str(tmp_path / "cpu_gemv.o")
        _run([f"{LLVM}/clang++", "-O2", "-std=c++17", "-fPIC", "-fopenmp", *SAN, f"-I{inc}", "-c",
              os.path.join(csrc, "cpu_gemv.cpp"), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(hip_obj, s) for s in b.SOURCES] + [ex.submit(cpu_obj)]
        objs = [f.result() for f in futs]
    lib = str(tmp_path / "libaqlm_san.so")
    _run([f"{LLVM}/clang++", "-shared", "-fPIC", *SAN, "-fopenmp", *objs, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/llvm/lib", "-o", lib])
    exe = str(tmp_path / "sanitize_check")
    _run([f"{LLVM}/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, f"-I{inc}",
          os.path.join(ROOT, "tests", "sanitize_check.c"), os.path.join(ROOT, "oracle", "aqlm_oracle.c"),
          f"-L{tmp_path}", "-laqlm_san", f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
          "-Wl,-rpath,/opt/rocm/llvm/lib", "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized checks failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "sanitized host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
