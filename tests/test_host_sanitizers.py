"""The host code of the C ABI (csrc/qdec_api.cpp) under AddressSanitizer,
LeakSanitizer and UndefinedBehaviorSanitizer. g++ builds that one file with
the sanitizers; the executable links it ahead of the built libqdec.so, whose
kernel launchers it calls, and runs tests/host_abi_checks.c: every
argument, config and lifecycle rejection that needs no GPU, host memory passed
as weights, and per-thread error text. The sanitizers end the run on any
invalid access, leak from the library's host code or undefined operation.
Leaks inside the ROCm runtime libraries themselves are suppressed."""
import os
import shutil
import subprocess

import pytest

from qwen3_kv_cache_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
SUPPRESS = ["libamdhip64", "libhsa-runtime64", "librocprofiler-register", "libhsakmt", "libdrm"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_abi_under_sanitizers(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not gxx or not gcc:
        pytest.skip("g++/gcc missing")
    if not os.path.exists(qbuild.LIB):
        pytest.skip("libqdec.so not built")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", qbuild.CSRC]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "drv.o", "abi_checks"))
    _run([gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), *inc, "-c",
          os.path.join(qbuild.CSRC, "qdec_api.cpp"), "-o", api_o])
    _run([gcc, "-std=c99", *SAN, "-Wall", "-Werror", *inc, "-c", os.path.join(ROOT, "tests", "host_abi_checks.c"),
          "-o", drv_o])
    libdir = os.path.dirname(qbuild.LIB)
    _run([gxx, *SAN, drv_o, api_o, qbuild.LIB, "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lpthread",
          f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    supp = tmp_path / "lsan.supp"
    supp.write_text("".join(f"leak:{lib}\n" for lib in SUPPRESS))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:strict_string_checks=1:detect_stack_use_after_return=1"
    env["LSAN_OPTIONS"] = f"suppressions={supp}:print_suppressions=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "host ABI checks passed" in r.stdout, out
    for marker in ("AddressSanitizer", "LeakSanitizer", "runtime error:"):
        assert marker not in out, out
