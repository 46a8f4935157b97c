"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/qoracle.c) with tests/sanitize/oracle_driver.c: every routine on small
  inputs and the pinned edge cases, with round-trip checks.
* The C ABI's host code -- argument validation in csrc/api.hip (sanitized on the host side
  only; its device code is built as usual) and the packed-weight blob parser csrc/blob.cpp --
  with tests/sanitize/abi_driver.cpp: every entry point given invalid or overflowing sizes
  (each call fails validation before anything is launched, so no GPU is needed) and 30,000
  randomly corrupted blobs.  The rest of the library is linked from its normal build.
Any sanitizer report ends the driver with a non-zero status."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_mixed_amd", "csrc")
OBJ = os.path.join(ROOT, "weight_only_mixed_amd", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", *SAN,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "qoracle.c"),
          "-o", exe, "-lm"])
    assert "oracle driver ok" in _run([exe], env=ENV)


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    others = sorted(f[:-4] for f in os.listdir(CSRC) if f.endswith(".hip") and f != "api.hip")  # the kernels
    if not all(os.path.exists(os.path.join(OBJ, o + ".o")) for o in others):
        _run(["python3", os.path.join(ROOT, "weight_only_mixed_amd", "build.py")])
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = str(tmp_path / "api_san.o")
    # host-side sanitizers only: each option follows -Xarch_host
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", *host_san, *inc, "-c", os.path.join(CSRC, "api.hip"), "-o", api])
    blob = str(tmp_path / "blob_san.o")
    _run(["g++", "-O1", "-g", "-std=c++17", *SAN, *inc, "-c", os.path.join(CSRC, "blob.cpp"), "-o", blob])
    drv = str(tmp_path / "drv.o")
    _run(["g++", "-O1", "-g", "-std=c++17", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          drv, api, blob, *[os.path.join(OBJ, o + ".o") for o in others], "-o", exe])
    assert "abi driver ok" in _run([exe], env=ENV)
