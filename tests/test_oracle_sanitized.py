"""The oracle's pin suite against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of ``oracle/oracle.c`` (host code only, on the CPU).

Memory errors and undefined behaviour in the oracle would not necessarily
change a pinned value; the sanitized build turns them into failures.  A
planted out-of-bounds write that every numeric pin misses shows that the
sanitizers are really active in the run.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from conftest import ROOT

import oracle
from test_oracle_mutants import PIN_FILES

SAN_FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fPIC",
             "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return path


def _build(tmpdir: str, name: str, text: str) -> str:
    src = os.path.join(tmpdir, f"{name}.c")
    lib = os.path.join(tmpdir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", *SAN_FLAGS, src, "-o", lib, "-lm", "-lpthread"], check=True,
                   capture_output=True)
    return lib


def _run_pins(lib: str, files) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in files]
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p",
                           "no:cacheprovider", *tests], env=env, capture_output=True, text=True,
                          cwd=ROOT, timeout=900)


def test_pins_pass_under_sanitizers(tmp_path):
    _runtime()
    lib = _build(str(tmp_path), "oracle_san", open(oracle.SRC_PATH).read())
    r = _run_pins(lib, PIN_FILES)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]


def test_sanitizers_catch_a_planted_overflow(tmp_path):
    """One word past the end of the per-sample word array: no pinned value
    changes, but the sanitized run must stop with a report."""
    _runtime()
    src = open(oracle.SRC_PATH).read()
    old = "for (int k = 0; k < OR_MAX_WORDS; ++k)"
    assert src.count(old) == 1
    lib = _build(str(tmp_path), "oracle_overflow", src.replace(old, old.replace("<", "<=")))
    r = _run_pins(lib, ["test_oracle_sampler.py"])
    out = r.stdout + r.stderr
    assert r.returncode != 0
    assert "runtime error" in out or "AddressSanitizer" in out, out[-3000:]
