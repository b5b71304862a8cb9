"""Shared test setup.

Markers: ``gpu`` tests need an AMD GPU and call the HIP library through its
C ABI; everything else runs on the CPU (oracle pins, host logic, library
load and exports).
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)
GOLDEN = os.path.join(TESTS, "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive checks that take tens of seconds")


def read_golden(name: str) -> list[list[str]]:
    """Rows of a golden text file, comments and blank lines dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def orc():
    """The oracle package, built if needed."""
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def torch_philox():
    """PyTorch's header Philox4x32-10 as a ctypes function (test-only helper)."""
    import ctypes
    try:
        import torch
    except Exception:  # pragma: no cover
        pytest.skip("torch headers unavailable")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    src = os.path.join(TESTS, "helpers", "torch_philox.cpp")
    lib = os.path.join(TESTS, "helpers", "libtorch_philox.so")
    if not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", f"-I{inc}", src,
                        "-o", lib + ".tmp"], check=True)
        os.replace(lib + ".tmp", lib)
    h = ctypes.CDLL(lib)
    h.ref_torch_philox_words.restype = None
    h.ref_torch_philox_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_void_p, ctypes.c_int64]

    def words(seed: int, subsequence: int, offset: int, count: int) -> np.ndarray:
        out = np.zeros(count, np.uint32)
        h.ref_torch_philox_words(seed, subsequence, offset, out.ctypes.data, count)
        return out

    return words
