"""ctypes binding of libfn_cpu.so: FusedNormalization on the host CPU with
SSE4.1 and F16C, the way page "(11) FusedNormalization" runs it (one image
per worker-thread call, fp32 SIMD arithmetic, F16C conversion, the erase
rectangle zeroed after the pass).

A host comparison path for measurements and tests, on numpy arrays in host
memory.  It is not a fallback for the GPU library: nothing in
``augmentation_amd.binding`` calls it.  Importing this module raises
ImportError if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfn_cpu.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                      f"g.build()'` from the repository root")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_lib.fn_cpu_fused_normalize.argtypes = [
    _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_float,
    ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
    ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, _P, _P, ctypes.c_int32]
_lib.fn_cpu_fused_normalize.restype = ctypes.c_int
_lib.fn_cpu_last_error.argtypes = []
_lib.fn_cpu_last_error.restype = ctypes.c_char_p

OUT_FP32, OUT_FP16, OUT_FP16_PAD4 = 0, 1, 2
EXPORTED = ("fn_cpu_fused_normalize", "fn_cpu_last_error")
PARAMS_DTYPE = np.dtype(
    [("flip", "<i4"), ("erase", "<i4"), ("i", "<i4"), ("j", "<i4"),
     ("eh", "<i4"), ("ew", "<i4"), ("attempt", "<i4"), ("words_used", "<i4")]
)


class FnCpuError(RuntimeError):
    pass


def fused_normalize(x: np.ndarray, mean, std, flip_p=0.5, erase_p=0.0, scale=(0.02, 0.33),
                    ratio=(0.3, 3.3), seed=0, out_dtype=OUT_FP32, first_sample_id=0,
                    threads=1, out: np.ndarray | None = None, with_params=False):
    """fn_cpu_fused_normalize on an (N, H, W, C) uint8 array; returns the
    output array (and the per-sample decisions when with_params)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    N, H, W, C = x.shape
    oc = 4 if out_dtype == OUT_FP16_PAD4 else C
    dt = np.float32 if out_dtype == OUT_FP32 else np.float16
    if out is None:
        out = np.empty((N, H, W, oc), dt)
    elif out.dtype != dt or out.shape != (N, H, W, oc) or not out.flags.c_contiguous:
        raise ValueError("out has the wrong shape, dtype or layout")
    m = (ctypes.c_float * C)(*np.broadcast_to(np.asarray(mean, np.float32), (C,)))
    s = (ctypes.c_float * C)(*np.broadcast_to(np.asarray(std, np.float32), (C,)))
    prm = np.zeros(N, PARAMS_DTYPE) if with_params else None
    rc = _lib.fn_cpu_fused_normalize(
        x.ctypes.data, N, H, W, C, m, s, flip_p, erase_p, scale[0], scale[1], ratio[0], ratio[1],
        seed & 0xFFFFFFFFFFFFFFFF, first_sample_id, out_dtype, out.ctypes.data,
        prm.ctypes.data if prm is not None else None, threads)
    if rc != 0:
        raise FnCpuError(_lib.fn_cpu_last_error().decode())
    return (out, prm) if with_params else out
