"""Host code under AddressSanitizer (with leak detection) and UBSan, on the CPU: the oracle
driven through decode, verify with skipped requests, the hand-off mode's near-tie counters
and the projection reference (tests/sanitize/oracle_driver.c); and the C-ABI host side
(kda_api.cpp, built with g++ for the host only and linked with the library's kernel
objects) through its validation paths, which return before any HIP call
(tests/sanitize/host_driver.c). GPU code is not instrumented."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module", autouse=True)
def _compilers():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc / g++ not available")


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-O1", "-g", *SAN, "-ffp-contract=off", "-I" + os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle under sanitizers: ok" in r.stdout


def test_host_abi_under_sanitizers(tmp_path):
    build = os.path.join(ROOT, "kimi_delta_attention_conv_amd", "_build")
    kernels = [o for o in sorted(glob.glob(os.path.join(build, "*.o"))) if "kda_api" not in o]
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not kernels or not os.path.isdir(os.path.join(rocm, "include", "hip")):
        pytest.skip("library objects not built (run __graft_entry__.build()) or no ROCm headers")
    csrc = os.path.join(ROOT, "kimi_delta_attention_conv_amd", "csrc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + csrc]
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "host_san")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I" + os.path.join(rocm, "include"), *inc, "-c", os.path.join(csrc, "kda_api.cpp"), "-o", api])
    _run(["gcc", "-std=c99", "-g", *SAN, *inc, "-c", os.path.join(HERE, "host_driver.c"), "-o", drv])
    _run(["g++", *SAN, "-o", exe, drv, api, *kernels, "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(rocm, "lib")])
    r = _run([exe], env=ENV, timeout=120)
    assert "host validation under sanitizers: ok" in r.stdout
