"""The library's host code (plan, validation, workspace sizing, status and
timing calls) built for the host only under AddressSanitizer and
UndefinedBehaviorSanitizer, and driven through the C ABI by
tests/host_check/abi_check.cpp. The driver's calls all fail validation or are
no-ops, so no kernel is launched (the device code is built as usual, without
sanitizers)."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "orthogonal_equivalence_cayley_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only (no device code is compiled)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def _build(out_dir):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    srcs.append(os.path.join(ROOT, "tests", "host_check", "abi_check.cpp"))

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, "-x", "hip", *FLAGS, *SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"{src}: {r.stderr[-2000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, srcs))
    exe = os.path.join(out_dir, "abi_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(r.stderr[-2000:])
    return exe


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = _build(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    sys.stdout.write(r.stdout[-4000:])
    sys.stderr.write(r.stderr[-4000:])
    if r.returncode == 77:
        pytest.skip("the driver runs only where no GPU is visible")
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "OK (0 failed checks)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
