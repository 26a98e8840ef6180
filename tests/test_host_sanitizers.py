"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host side (the CLOCK residency table, the host record encoder and
f64 -> f16 rounding, the size helpers and every entry point's argument checks,
all in csrc/kv_api.hip) is compiled with -fsanitize=address,undefined for the host
(device code as usual), linked with the library's other objects into the driver
tests/host_sanitize/host_checks.cpp, and run. The driver exits non-zero on a failed
check; a sanitizer report aborts it. No GPU is used: the driver only calls host code
paths, and the entry points with arguments they reject before enqueuing anything.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
BUILD = os.path.join(ROOT, "offloaded_kv_cache_amd", "_build")
OTHERS = ["kv_decode.o", "kv_append.o", "kv_gather.o", "kv_select.o"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not available")
    objs = [os.path.join(BUILD, o) for o in OTHERS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (offloaded_kv_cache_amd/build.py)")
    api = os.path.join(tmp_path, "kv_api_san.o")
    drv = os.path.join(tmp_path, "host_checks.o")
    exe = os.path.join(tmp_path, "host_checks")
    inc = "-I" + os.path.join(ROOT, "include")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, inc,
          "-c", os.path.join(ROOT, "offloaded_kv_cache_amd", "csrc", "kv_api.hip"), "-o", api])
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", inc, "-c", os.path.join(ROOT, "tests", "host_sanitize", "host_checks.cpp"),
          "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, drv, api, *objs])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env, cwd=tmp_path)
    assert r.returncode == 0 and "host checks passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
