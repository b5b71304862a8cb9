"""CPU oracle for FusedNormalization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library
and its binding in ``augmentation_amd``) never imports, links or calls it,
and this package imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C loops); this module only
marshals numpy arrays through ctypes.  Every function cites, in the C
source, the passage of the page "(11) FusedNormalization"
(tech-renaissance.cn/blog/?p=487) that it follows.

Pinning: every function here is pinned by ``tests/test_oracle_*.py``
against known-answer vectors, closed forms, exact rational arithmetic,
library routines and brute force.  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
BUILT_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB lets the mutation test load a deliberately broken copy.
LIB_PATH = os.environ.get("ORACLE_LIB") or BUILT_LIB
SRC_PATH = os.path.join(_HERE, "oracle.c")

# gcc flags: -ffp-contract=off keeps every fp32 operation of the sampler a
# separately rounded IEEE operation, as the page's float code is written.
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-Wall", "-Wextra", "-shared"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    cmd = ["gcc", *CFLAGS, SRC_PATH, "-o", BUILT_LIB + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BUILT_LIB + ".tmp", BUILT_LIB)
    return BUILT_LIB


PARAMS_DTYPE = np.dtype(
    [("flip", "<i4"), ("erase", "<i4"), ("i", "<i4"), ("j", "<i4"),
     ("eh", "<i4"), ("ew", "<i4"), ("attempt", "<i4"), ("words_used", "<i4")]
)
MAX_WORDS = 24

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    u32, u64, i32, i64, f32 = (ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32,
                               ctypes.c_int64, ctypes.c_float)
    sigs = {
        "or_philox4x32_10": (None, [P, P, P]),
        "or_word": (u32, [u64, u64, u64]),
        "or_u01": (f32, [u32]),
        "or_randint": (i32, [i32, i32, u32]),
        "or_log_ratio": (f32, [f32]),
        "or_expf": (f32, [f32]),
        "or_erase_dims": (ctypes.c_int, [u32, u32, i32, i32, f32, f32, f32, f32, P, P]),
        "or_params_from_words": (ctypes.c_int, [P, i64, i32, i32, f32, f32, f32, f32, f32, f32, P]),
        "or_params": (None, [u64, i64, i64, i32, i32, f32, f32, f32, f32, f32, f32, P]),
        "or_apply": (None, [P, i64, i32, i32, i32, P, P, P, P]),
        "or_fused_normalize": (ctypes.c_int, [P, i64, i64, i32, i32, i32, P, P, f32, f32, f32, f32,
                                              f32, f32, u64, P, ctypes.c_int]),
        "or_expf_array": (None, [P, i64, P]),
        "or_erase_dims_array": (None, [P, P, i64, i32, i32, f32, f32, f32, f32, P, P, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _f32(x) -> float:
    """The fp32 value of x (arguments cross the C ABI as float)."""
    return float(np.float32(x))


# ----------------------------------------------------------------- generator

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.zeros(4, np.uint32)
    _load().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def word(seed: int, n: int, k: int) -> int:
    return int(_load().or_word(seed, n, k))


def words(seed: int, n: int, count: int = MAX_WORDS) -> np.ndarray:
    return np.array([word(seed, n, k) for k in range(count)], dtype=np.uint32)


def u01(w: int) -> float:
    return float(_load().or_u01(w))


def randint(lo: int, hi: int, w: int) -> int:
    return int(_load().or_randint(lo, hi, w))


def log_ratio(r: float) -> float:
    return float(_load().or_log_ratio(_f32(r)))


def expf(L: float) -> float:
    return float(_load().or_expf(_f32(L)))


def expf_array(L: np.ndarray) -> np.ndarray:
    L = np.ascontiguousarray(L, dtype=np.float32)
    out = np.empty_like(L)
    _load().or_expf_array(_ptr(L), L.size, _ptr(out))
    return out


# ------------------------------------------------------------------- sampler

def erase_dims(w_scale: int, w_ratio: int, H: int, W: int, scale=(0.02, 0.33),
               ratio=(0.3, 3.3)):
    """(eh, ew, accepted) of one attempt from its two words."""
    eh = ctypes.c_int32()
    ew = ctypes.c_int32()
    ok = _load().or_erase_dims(w_scale, w_ratio, H, W, _f32(scale[0]), _f32(scale[1]),
                               log_ratio(ratio[0]), log_ratio(ratio[1]),
                               ctypes.byref(eh), ctypes.byref(ew))
    return eh.value, ew.value, bool(ok)


def erase_dims_array(w_scale: np.ndarray, w_ratio: np.ndarray, H: int, W: int,
                     scale=(0.02, 0.33), ratio=(0.3, 3.3)):
    ws = np.ascontiguousarray(w_scale, dtype=np.uint32)
    wr = np.ascontiguousarray(w_ratio, dtype=np.uint32)
    assert ws.shape == wr.shape
    eh = np.empty(ws.shape, np.int32)
    ew = np.empty(ws.shape, np.int32)
    acc = np.empty(ws.shape, np.uint8)
    _load().or_erase_dims_array(_ptr(ws), _ptr(wr), ws.size, H, W, _f32(scale[0]),
                                _f32(scale[1]), _f32(ratio[0]), _f32(ratio[1]),
                                _ptr(eh), _ptr(ew), _ptr(acc))
    return eh, ew, acc.astype(bool)


def params_from_words(stream, H: int, W: int, flip_p: float, erase_p: float,
                      scale=(0.02, 0.33), ratio=(0.3, 3.3)) -> np.ndarray:
    """Parameters of one sample from an explicit word stream (None if too short)."""
    w = np.ascontiguousarray(stream, dtype=np.uint32)
    out = np.zeros(1, PARAMS_DTYPE)
    rc = _load().or_params_from_words(_ptr(w), w.size, H, W, _f32(flip_p), _f32(erase_p),
                                      _f32(scale[0]), _f32(scale[1]), log_ratio(ratio[0]),
                                      log_ratio(ratio[1]), _ptr(out))
    return None if rc != 0 else out[0]


def params(seed: int, first_n: int, count: int, H: int, W: int, flip_p: float,
           erase_p: float, scale=(0.02, 0.33), ratio=(0.3, 3.3)) -> np.ndarray:
    out = np.zeros(count, PARAMS_DTYPE)
    _load().or_params(seed, first_n, count, H, W, _f32(flip_p), _f32(erase_p), _f32(scale[0]),
                      _f32(scale[1]), _f32(ratio[0]), _f32(ratio[1]), _ptr(out))
    return out


# --------------------------------------------------------------------- pixels

def _mean_std(mean, std, C):
    m = np.ascontiguousarray(np.broadcast_to(np.asarray(mean, np.float32), (C,)), np.float32)
    s = np.ascontiguousarray(np.broadcast_to(np.asarray(std, np.float32), (C,)), np.float32)
    return m, s


def apply(x: np.ndarray, mean, std, prm: np.ndarray) -> np.ndarray:
    """Output of a batch (N,H,W,C) uint8 given per-sample parameters."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    N, H, W, C = x.shape
    prm = np.ascontiguousarray(prm, dtype=PARAMS_DTYPE)
    assert prm.shape == (N,)
    m, s = _mean_std(mean, std, C)
    out = np.empty(x.shape, np.float32)
    _load().or_apply(_ptr(x), N, H, W, C, _ptr(m), _ptr(s), _ptr(prm), _ptr(out))
    return out


def fused_normalize(x: np.ndarray, mean, std, flip_p: float, erase_p: float,
                    scale=(0.02, 0.33), ratio=(0.3, 3.3), seed: int = 0, first_n: int = 0,
                    threads: int = 1):
    """The whole operation on images first_n .. first_n+len(x)-1 of a batch.

    Returns (fp32 output, threads used)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    N, H, W, C = x.shape
    m, s = _mean_std(mean, std, C)
    out = np.empty(x.shape, np.float32)
    used = _load().or_fused_normalize(_ptr(x), first_n, N, H, W, C, _ptr(m), _ptr(s),
                                      _f32(flip_p), _f32(erase_p), _f32(scale[0]),
                                      _f32(scale[1]), _f32(ratio[0]), _f32(ratio[1]), seed,
                                      _ptr(out), threads)
    return out, int(used)
