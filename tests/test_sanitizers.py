"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with g++ -fsanitize=address,undefined and run here:
  * the C-ABI front end (csrc/fa_api.cpp) linked against host stand-ins of
    the HIP calls and kernel launchers (tests/sanitize/abi_stubs.cpp), driven
    through every entry point of include/fa.h with valid and invalid
    arguments on real host buffers; the stand-in launchers check that every
    workspace region lies inside the caller's workspace;
  * the fp64 oracle (oracle/attention_oracle.cpp) on small problems with
    exactly sized buffers (fixed and packed layouts with an empty sequence,
    masks, GQA, dropout, row / head selections).
Any out-of-bounds access, use after free, signed overflow or other undefined
behaviour ends the program with a sanitizer report.  No GPU and no device
code are involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _have_sanitizers(tmp):
    src = tmp / "probe.cpp"
    src.write_text("int main() { return 0; }\n")
    r = subprocess.run(["g++", *SAN, str(src), "-o", str(tmp / "probe")], capture_output=True)
    return r.returncode == 0


@pytest.fixture(scope="module")
def tmp(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    if shutil.which("g++") is None or not _have_sanitizers(d):
        pytest.skip("g++ with AddressSanitizer/UBSan not available")
    return d


def _build_and_run(tmp, name, sources, extra):
    exe = str(tmp / name)
    subprocess.run(["g++", "-std=c++17", *SAN, *extra, *sources, "-o", exe, "-pthread"], check=True,
                   capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    return r.stdout


def test_c_abi_front_end_under_sanitizers(tmp):
    csrc = os.path.join(ROOT, "exact_tiled_attention_10_amd", "csrc")
    out = _build_and_run(tmp, "abi", [os.path.join(csrc, "fa_api.cpp"),
                                      os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
                                      os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")],
                         ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")])
    assert "abi: all checks passed" in out


def test_oracle_under_sanitizers(tmp):
    out = _build_and_run(tmp, "oracle", [os.path.join(ROOT, "oracle", "attention_oracle.cpp"),
                                         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp")], [])
    assert "oracle: all checks passed" in out
