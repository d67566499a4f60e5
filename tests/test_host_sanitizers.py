"""The host code of the C ABI (argument validation, buffer sizing, split
planning) and the CPU oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU.

`tests/sanitize/host_checks.c` drives every validation path that returns
before a launch and the oracle's functions on small, exactly sized inputs;
the kernel launchers are linked as stubs that abort if reached, which also
checks that validation precedes every launch.  Host code only: the device
side of the HIP translation unit is built without sanitizers (`-Xarch_host`
puts each sanitizer flag on the host compilation alone).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_cache_05_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-8000:])
    return r


@pytest.mark.timeout(600)
def test_host_code_and_oracle_under_sanitizers(tmp_path):
    for tool in (HIPCC, CLANG, CLANGXX):
        if not os.path.exists(tool):
            pytest.skip("%s not found" % tool)
    hip = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-gpu-rdc",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *HOST_SAN]
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "host_checks")
    _run([*hip, "-x", "hip", "-c", os.path.join(CSRC, "kvq_api.cpp"), "-o", api])
    _run([*hip, "-x", "hip", "-c", os.path.join(HERE, "launch_stubs.cpp"), "-o", stubs])
    _run([CLANG, "-O1", "-g", "-std=c11", *SAN, "-I" + os.path.join(ROOT, "include"),
          "-I" + os.path.join(ROOT, "oracle"), "-c", os.path.join(HERE, "host_checks.c"), "-o", drv])
    _run([CLANGXX, *SAN, drv, api, stubs, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm", "-o", exe])
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    r = _run([exe], env=env, timeout=300)
    assert "host checks passed" in r.stdout
