"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two drivers in tests/sanitize/ are built here with the sanitizers and run on
the CPU (no GPU is touched):

* host_api_driver.cpp with the library's host-only sources -- the C ABI's
  validation, workspace sizing and path choice (api.cpp, sizing.cpp) and the
  block-format packer (pack_blocks.cpp); the kernel launchers are stubs that
  count calls, and every call made returns before a launch;
* oracle_driver.c with oracle/oracle.c (fp16 conversions, the b-bit
  quantizer, route and layer in every expert format).

Each driver uses exact-size heap buffers, so an out-of-bounds access in the
code under test is reported; undefined behaviour aborts (no recovery). The
sanitizers apply to host code only (every sanitizer flag on a hipcc line goes
through -Xarch_host; the HIP sources are compiled for the host side only).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_decode_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_ONLY = ["-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_sanitizers(tmp_path):
    objs = []
    for src, extra in ((os.path.join(HERE, "host_api_driver.cpp"), []), (os.path.join(CSRC, "api.cpp"), []),
                       (os.path.join(CSRC, "sizing.cpp"), []),
                       (os.path.join(CSRC, "pack_blocks.cpp"), ["-ffp-contract=off"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *HOST_ONLY, *SAN, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_api_driver")
    _run([HIPCC, *SAN, "-o", exe, *objs])
    r = _run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout
