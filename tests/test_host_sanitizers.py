"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every library source with ASan and UBSan on the host side only (the
device code is compiled as usual, unsanitised, and never runs here), links tests/host_sanitize/driver.cpp against it, and runs
the driver: configuration and argument validation, blob sizes, the GEMM tile
planner over a sweep of shapes, the log-mel filter tables and the per-thread
error messages, all without a GPU.  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "whisper_audio_encoder_amd", "csrc")
SOURCES = ["gemm.hip", "attention.hip", "layernorm.hip", "frontend.hip", "xattn.hip", "argmax.hip", "wenc_runtime.cpp"]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.timeout(600)
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    procs = []
    objs = []
    for src in SOURCES + [os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")]:
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.basename(path) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *FLAGS, *SAN, "-c", path, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=500)
        assert p.returncode == 0, err
    exe = str(tmp_path / "driver")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, *objs, "-lpthread"], timeout=300)
    env = dict(os.environ)
    # the HIP runtime's own allocations are not this library's to free
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "host checks passed" in r.stdout
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
