"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

* The C ABI: every csrc/*.hip file is compiled with the sanitizers on its host side
  only (device code is unchanged) and linked with tests/sanitize/abi_driver.cpp,
  which sweeps the configuration check, the workspace layout for extreme sizes and
  every entry point's argument checks up to the kernel launch (which fails with
  QSA_ERR_HIP where there is no GPU).
* The CPU oracle (oracle/qsa_oracle.c and the all-core timing form) with
  tests/sanitize/oracle_driver.c, on small and degenerate inputs, leak checks on.

A sanitizer report aborts the driver, and the test fails with its output.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_decode_qsa_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/bin/amdclang++"
# host-side sanitizers only: each -fsanitize is scoped to the host compilation
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm")
def test_abi_host_code_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_HOST,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        run([HIPCC, *flags, "-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_driver.o")
    run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
         os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_sweep")
    run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, "-o", exe, drv, *objs])
    # the HIP runtime keeps its allocations until exit: leak checks are for the oracle
    r = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"), timeout=300)
    assert "abi sweep: ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sweep")
    run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-pthread", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "qsa_oracle.c"),
         os.path.join(ROOT, "oracle", "qsa_oracle_mt.c"), "-lm"])
    r = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert "oracle sweep: ok" in r.stdout
