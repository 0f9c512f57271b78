"""The C ABI's host code (argument validation, planning, workspace layout,
the launch-shape helpers) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (the GPU code is unchanged),
driven by tests/abi_sanitize/harness.cpp over extreme and random arguments.
Every call there is host-only or fails validation before any device work, so
this runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_layer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# sanitizers on the host half of each compile only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    import concurrent.futures as cf
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(ROOT, "tests", "abi_sanitize", "harness.cpp"))

    def compile_one(src):
        obj = os.path.join(tmp_path, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        r = subprocess.run([HIPCC, *FLAGS, *SAN, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(tmp_path, "abi_harness")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "abi sanitize harness: ok" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
