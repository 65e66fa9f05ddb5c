"""The oracle's pin suite under AddressSanitizer and UndefinedBehaviorSanitizer
(host only): oracle.c is built with -fsanitize=address,undefined (every
report fatal), the pin tests run in a child process against that build, and
any out-of-bounds access, leak-free misuse or undefined operation in the
oracle fails this test."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no ASan runtime for gcc here")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                        "-fsanitize=address,undefined",
                                                        "-fno-sanitize-recover=all"]
    subprocess.check_call(["gcc", *flags, os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib,
                           "-lm"])
    env = dict(os.environ)
    env["ORACLE_LIB"] = lib
    env["LD_PRELOAD"] = " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    # the interpreter itself is not instrumented: its allocations are not the oracle's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_glu.py"),
                        os.path.join(ROOT, "tests", "test_oracle_gate.py"),
                        os.path.join(ROOT, "tests", "test_oracle_mlgru.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no ASan runtime for gcc here")
def test_sanitized_run_catches_a_planted_overrun(tmp_path):
    """A copy of the oracle whose activation copy runs one element past its
    buffer: the same sanitized pin run must stop with an AddressSanitizer
    report (so the run above is really checked)."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    slip = "for (int64_t i = 0; i < M * K; ++i) A[i] = xq[i];"
    assert slip in src
    bad = tmp_path / "oracle_overrun.c"
    bad.write_text(src.replace(slip, slip.replace("i < M * K", "i <= M * K"), 1))
    lib = str(tmp_path / "liboracle_overrun.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-I", os.path.join(ROOT, "oracle"), "-std=c11",
                           "-shared", "-fPIC", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", str(bad), "-o", lib, "-lm"])
    env = dict(os.environ, ORACLE_LIB=lib, ASAN_OPTIONS="detect_leaks=0",
               LD_PRELOAD=" ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stdout + r.stderr
