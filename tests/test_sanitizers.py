"""CPU sanitizer job: the oracle and the host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.

* The oracle (oracle/sgqa_oracle.c) is compiled with gcc together with tests/sanitize/oracle_driver.c,
  which runs every oracle function on small inputs and edge cases (N < B, one-token sequences,
  B = 1 and 64, k covering the context, row subsets, FP8 codes).
* The library's host code is compiled with the sanitizers (hipcc, sanitizer flags for the host
  only; the device code is built unoptimised, as it never runs here) and linked with
  tests/sanitize/abi_driver.cpp, which drives every entry point and sgqa_workspace_size through
  their validation paths, extreme sizes included. No call in it is valid, so nothing is launched.
Any sanitizer report aborts the driver (-fno-sanitize-recover=all) and fails the test. Nothing here
needs a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_sparse_long_sgqa_amd", "csrc")
SOURCES = ["sgqa_api", "compress", "index_topk", "decode_select", "union", "attend", "attend_bwd"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    rc, out = run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=all", "-ffp-contract=off", "-fopenmp", "-Wall", "-Wextra", "-o", exe,
                   os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "sgqa_oracle.c"), "-lm"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    rc, out = run([exe], env=env, timeout=600)
    assert rc == 0 and "Sanitizer" not in out, out
    assert "ran clean" in out


def test_host_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    common = ["-std=c++17", "-g", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I" + os.path.join(ROOT, "include")]
    procs, objs = [], []
    for name in SOURCES:
        obj = str(tmp_path / f"{name}.o")
        objs.append(obj)
        cmd = [HIPCC, "--offload-arch=gfx950", "-Xarch_device", "-O0", "-Xarch_host", "-O1", *common, *SAN_HOST,
               "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out
    drv = str(tmp_path / "abi_driver.o")
    rc, out = run([HIPCC, "-x", "c++", "-O1", "-g", "-std=c++17", *SAN_HOST, "-I" + os.path.join(ROOT, "include"),
                   "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "abi_driver")
    rc, out = run([HIPCC, "--offload-arch=gfx950", *SAN_HOST[:4], "-o", exe, drv, *objs])
    assert rc == 0, out
    # The HIP runtime is not instrumented and keeps allocations until exit: no leak report.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = run([exe], env=env, timeout=600)
    assert rc == 0 and "Sanitizer" not in out and "runtime error" not in out, out
    assert "rejected cleanly" in out
