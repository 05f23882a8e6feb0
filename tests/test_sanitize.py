"""Sanitizer builds on the CPU: the oracle (plain C) and the library's host
lookup-table parser, built with AddressSanitizer and UndefinedBehaviorSanitizer
(any report aborts), run over small seeded problems and malformed tables."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd_build, exe, args=()):
    subprocess.check_call(cmd_build)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: " not in r.stderr, \
        r.stdout[-2000:] + r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    out = _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "oracle_harness.c"),
                os.path.join(ROOT, "oracle", "bsa_ref.c"), "-o", exe, "-lm"], exe)
    assert "oracle harness ok" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_lut_parser_under_sanitizers(tmp_path):
    from block_sparse_attention_08_amd import build
    build.write_lut_include()
    csrc = os.path.join(ROOT, "block_sparse_attention_08_amd", "csrc")
    exe = str(tmp_path / "lut_harness")
    out = _run(["g++", "-std=c++17", *SAN, "-I", csrc, "-I", os.path.join(ROOT, "include"),
                os.path.join(HERE, "lut_harness.cpp"), os.path.join(csrc, "bsa_lut.cpp"), "-o", exe],
               exe, [build.LUT])
    assert "lut harness ok" in out
