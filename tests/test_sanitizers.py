"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the library's
host side (argument validation and size queries of every entry point, built with the
sanitizers on the host pass only) and the CPU oracle (every entry point on a small seeded
layer), each driven by a small C program (tests/sanitize/) that fails on any report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert p.returncode == 0, (" ".join(cmd), p.stdout[-3000:], p.stderr[-3000:])
    return p


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("san"))


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang")
def test_library_host_code_under_sanitizers(outdir):
    sys.path.insert(0, ROOT)
    from bit_quantized_expert_top_amd import build as hip_build
    lib = hip_build.build(sanitize=True, out=os.path.join(outdir, "libmoeq4_san.so"))
    exe = os.path.join(outdir, "abi_check")
    _run([CLANG, *SAN, "-o", exe, os.path.join(HERE, "abi_check.c"), lib,
          f"-Wl,-rpath,{outdir}", "-Wl,-rpath,/opt/rocm/lib"])
    p = _run([exe], env=ENV)
    assert "abi_check ok" in p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(outdir):
    exe = os.path.join(outdir, "oracle_check")
    _run(["gcc", "-O1", "-fopenmp", "-ffp-contract=off", "-std=c11", *SAN, "-o", exe,
          os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    p = _run([exe], env=ENV)
    assert "oracle_check ok" in p.stdout
