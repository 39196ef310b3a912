"""The C-ABI front end under host AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every library source and tests/abi_sanitize_driver.cpp with hipcc,
the sanitizers on the host side only (device code is built as usual and never
launched), links one executable and runs it: every entry point is called with
arguments the boundary must reject and every size query with extreme values.
A memory error, an overflow of signed arithmetic or a wrong status fails the
test.  No GPU is needed: every call in the driver is rejected before a device
call could reach a kernel."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_int4_gemm_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_under_host_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    flags = ["-xhip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SAN]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    srcs.append(os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([hipcc, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, f"hipcc failed on {src}:\n{res.stderr[-4000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_sanitize_driver")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, f"link failed:\n{res.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, f"driver failed (rc={run.returncode}):\n{run.stdout}\n{run.stderr[-6000:]}"
    assert "all checks passed" in run.stdout
