"""The host runtime (handle planning, workspace carving, argument checks,
sampler schedules, training parameter layout, packed-sequence planning) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.cpp and train_api.cpp are compiled with both sanitizers on their host
side only (each -fsanitize= behind -Xarch_host; the device code is not
instrumented), linked with the uninstrumented kernel objects into a separate
library, and driven by tests/host_runtime_driver.c, which calls every entry
point that works on the host over the workloads' configurations.  A
sanitizer report or a failed check fails the test."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host_runtime_driver.c")
HOST_SOURCES = ("api.cpp", "train_api.cpp")
CLANG = "/opt/rocm/llvm/bin/clang"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}")
    return res


@pytest.mark.timeout(600)
def test_host_runtime_under_address_and_ub_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists(CLANG):
        pytest.skip("ROCm toolchain not found")
    from diffusion_transformer_denoiser_amd import build as B

    objs = []
    for src in B.SOURCES:
        obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        if src in HOST_SOURCES:
            obj = str(tmp_path / (os.path.splitext(src)[0] + "_san.o"))
            _run([hipcc, "-x", "hip", *B.common_flags(), "-O1", "-g",
                  "-Xarch_host", "-fsanitize=address,undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer",
                  "-c", os.path.join(B.CSRC, src), "-o", obj])
        elif not os.path.exists(obj):
            os.makedirs(B.BUILD, exist_ok=True)
            obj = B.compile_one(src)
        objs.append(obj)
    lib = str(tmp_path / "libdit_san.so")
    # the sanitizer runtime comes with the driver executable below
    _run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    exe = str(tmp_path / "host_runtime_driver")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), DRIVER,
          "-L", str(tmp_path), "-ldit_san", f"-Wl,-rpath,{tmp_path}",
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe])
    supp = tmp_path / "lsan.supp"
    # allocations the HIP runtime keeps until exit are not this library's
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler\n")
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:detect_stack_use_after_return=1",
               LSAN_OPTIONS=f"suppressions={supp}:print_suppressions=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " 0 failed" in res.stdout
