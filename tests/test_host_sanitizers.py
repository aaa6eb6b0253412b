"""Host code of the C-ABI layer (argument validation, pool geometry, workspace
sizing, split choice) and of the rotation fit, built with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only; the device code of those
files is compiled as usual and never run) and exercised by a driver
(tests/host_sanitize_driver.cpp) whose kernel launchers are stubs. Any
sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "looped_transformer_decode_rq_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def _tool(name):
    for c in (os.path.join("/opt/rocm/bin", name), os.path.join("/opt/rocm/llvm/bin", name), shutil.which(name)):
        if c and os.path.exists(c):
            return c
    pytest.skip(f"{name} not found")


def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = _tool("hipcc"), _tool("amdclang++")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC]
    objs = []
    for src in ("rq_api.cpp", "rq_fit.cpp", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        r = subprocess.run([hipcc, *common, *san, "-x", "hip", "-c", path, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "host_sanitize")
    link = [clang, "-fsanitize=address,undefined", *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all checks passed" in out
