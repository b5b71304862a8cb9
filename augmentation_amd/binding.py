"""ctypes binding of libfn.so: the C entry points under the same names.

Argument marshalling only: every step of the operation runs in the
library's HIP kernels.  PyTorch supplies device memory and streams; a
buffer argument may be a torch CUDA tensor (its data pointer is passed) or
a raw device address as an int.  A nonzero return code raises ``FnError``
with the library's message.  Importing this module raises ImportError if
the library has not been built (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                      f"g.build()'` from the repository root")

_lib = ctypes.CDLL(LIB_PATH)

FN_OK, FN_EINVAL, FN_EOVERFLOW, FN_EHIP = 0, -1, -2, -3
FN_OUT_FP32, FN_OUT_FP16, FN_OUT_FP16_PAD4 = 0, 1, 2

# fn_sample_params: eight int32 fields, 32 bytes
PARAMS_DTYPE = np.dtype(
    [("flip", "<i4"), ("erase", "<i4"), ("i", "<i4"), ("j", "<i4"),
     ("eh", "<i4"), ("ew", "<i4"), ("attempt", "<i4"), ("words_used", "<i4")]
)

_P = ctypes.c_void_p
_u64, _i64, _i32, _f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "fn_fused_normalize": [_P, _i64, _i32, _i32, _i32, _P, _P, _f32, _f32, _f32, _f32, _f32, _f32,
                           _u64, _i32, _P, _P],
    "fn_fused_normalize_ex": [_P, _i64, _i64, _i64, _i32, _i32, _i32, _P, _P, _f32, _f32, _f32,
                              _f32, _f32, _f32, _u64, _i64, _i32, _P, _P],
    "fn_params": [_u64, _i64, _i32, _i32, _f32, _f32, _f32, _f32, _f32, _f32, _P, _P],
    "fn_params_ex": [_u64, _i64, _i64, _i32, _i32, _f32, _f32, _f32, _f32, _f32, _f32, _P, _P],
    "fn_test_erase_dims": [_P, _P, _i64, _i32, _i32, _f32, _f32, _f32, _f32, _P, _P, _P, _P],
    "fn_test_cr_ops": [_i32, _P, _P, _i64, _P, _P],
    "fn_test_stream": [_P, _P, _i64, _i32, _P],
    "fn_test_timeline": [_P, _i64],
}


def _declare(lib) -> None:
    for name, args in _SIGS.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    lib.fn_last_error.argtypes = []
    lib.fn_last_error.restype = ctypes.c_char_p


_declare(_lib)

EXPORTED = ("fn_fused_normalize", "fn_fused_normalize_ex", "fn_params", "fn_params_ex",
            "fn_last_error", "fn_test_erase_dims", "fn_test_cr_ops", "fn_test_stream",
            "fn_test_timeline")

TIMELINE_LIB_PATH = os.path.join(_HERE, "libfn_timeline.so")


def timeline_library():
    """The instrumented build libfn_timeline.so (same entry points; its
    tiles kernel records per-tile clock stamps, see fn_test_timeline), as a
    ctypes handle.  A measurement tool: the product path is libfn.so."""
    if not os.path.exists(TIMELINE_LIB_PATH):
        raise ImportError(f"{TIMELINE_LIB_PATH} is not built")
    lib = ctypes.CDLL(TIMELINE_LIB_PATH)
    _declare(lib)
    return lib


class FnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libfn error {code}: {message}")
        self.code = code


def fn_last_error() -> str:
    return _lib.fn_last_error().decode()


def _addr(x) -> int | None:
    """Device address of a torch tensor or an int (None/0 -> NULL)."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(rc: int) -> int:
    if rc != FN_OK:
        raise FnError(rc, fn_last_error())
    return rc


_FLOATS: dict = {}  # recent constant arrays: the library only reads them during the call


def _host_floats(v, C: int):
    try:
        key = (C, v if isinstance(v, tuple) else tuple(v) if hasattr(v, "__len__") else v)
        a = _FLOATS.get(key)
        if a is not None:
            return a
    except TypeError:  # unhashable values
        key = None
    a = (ctypes.c_float * C)()
    vals = list(v) if hasattr(v, "__len__") else [v] * C
    if len(vals) != C:
        raise ValueError(f"expected {C} values, got {len(vals)}")
    for k, x in enumerate(vals):
        a[k] = float(x)
    if key is not None and len(_FLOATS) < 64:
        _FLOATS[key] = a
    return a


def fn_fused_normalize(in_u8, N, H, W, C, mean, std, flip_p, erase_p, scale_min, scale_max,
                       ratio_min, ratio_max, seed, out_dtype, out, stream=None) -> int:
    return _check(_lib.fn_fused_normalize(
        _addr(in_u8), N, H, W, C, _host_floats(mean, C), _host_floats(std, C), flip_p, erase_p,
        scale_min, scale_max, ratio_min, ratio_max, seed & 0xFFFFFFFFFFFFFFFF, out_dtype,
        _addr(out), _stream(stream)))


def fn_fused_normalize_ex(in_u8, in_row_stride, in_image_stride, N, H, W, C, mean, std, flip_p,
                          erase_p, scale_min, scale_max, ratio_min, ratio_max, seed,
                          first_sample_id, out_dtype, out, stream=None) -> int:
    return _check(_lib.fn_fused_normalize_ex(
        _addr(in_u8), in_row_stride, in_image_stride, N, H, W, C, _host_floats(mean, C),
        _host_floats(std, C), flip_p, erase_p, scale_min, scale_max, ratio_min, ratio_max,
        seed & 0xFFFFFFFFFFFFFFFF, first_sample_id, out_dtype, _addr(out), _stream(stream)))


def fn_params_ex(seed, first_sample_id, N, H, W, flip_p, erase_p, scale_min, scale_max,
                 ratio_min, ratio_max, params_dev, stream=None) -> int:
    return _check(_lib.fn_params_ex(seed & 0xFFFFFFFFFFFFFFFF, first_sample_id, N, H, W, flip_p,
                                    erase_p, scale_min, scale_max, ratio_min, ratio_max,
                                    _addr(params_dev), _stream(stream)))


def fn_params(seed, N, H, W, flip_p, erase_p, scale_min, scale_max, ratio_min, ratio_max,
              params_dev, stream=None) -> int:
    return _check(_lib.fn_params(seed & 0xFFFFFFFFFFFFFFFF, N, H, W, flip_p, erase_p, scale_min,
                                 scale_max, ratio_min, ratio_max, _addr(params_dev),
                                 _stream(stream)))


def fn_test_erase_dims(w_scale, w_ratio, count, H, W, scale_min, scale_max, ratio_min, ratio_max,
                       eh, ew, accepted, stream=None) -> int:
    return _check(_lib.fn_test_erase_dims(_addr(w_scale), _addr(w_ratio), count, H, W, scale_min,
                                          scale_max, ratio_min, ratio_max, _addr(eh), _addr(ew),
                                          _addr(accepted), _stream(stream)))


def fn_test_cr_ops(op, a, b, count, out, stream=None) -> int:
    return _check(_lib.fn_test_cr_ops(op, _addr(a), _addr(b), count, _addr(out), _stream(stream)))


def fn_test_stream(src, dst, in_bytes, widen, stream=None) -> int:
    return _check(_lib.fn_test_stream(_addr(src), _addr(dst), in_bytes, widen, _stream(stream)))


def fn_test_timeline(stamps, tiles) -> int:
    """libfn.so records no timeline: this raises FnError (FN_EINVAL)."""
    return _check(_lib.fn_test_timeline(_addr(stamps), tiles))


# ------------------------------------------------------------ tensor helpers

def fused_normalize(x: torch.Tensor, mean, std, flip_p=0.5, erase_p=0.0, scale=(0.02, 0.33),
                    ratio=(0.3, 3.3), seed=0, out_dtype=FN_OUT_FP32, out=None,
                    stream=None) -> torch.Tensor:
    """fn_fused_normalize on an (N, H, W, C) uint8 CUDA tensor; returns (or
    fills) the (N, H, W, C) float32/float16 output tensor, (N, H, W, 4)
    float16 for FN_OUT_FP16_PAD4."""
    if x.dtype != torch.uint8 or x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous (N, H, W, C) uint8 CUDA tensor")
    N, H, W, C = x.shape
    tdt = torch.float32 if out_dtype == FN_OUT_FP32 else torch.float16
    shape = (N, H, W, 4 if out_dtype == FN_OUT_FP16_PAD4 else C)
    if out is None:
        out = torch.empty(shape, dtype=tdt, device=x.device)
    elif out.dtype != tdt or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of shape %s and out_dtype" % (shape,))
    fn_fused_normalize(x, N, H, W, C, mean, std, flip_p, erase_p, scale[0], scale[1], ratio[0],
                       ratio[1], seed, out_dtype, out, stream)
    return out


def sample_params(N, H, W, flip_p=0.5, erase_p=0.0, scale=(0.02, 0.33), ratio=(0.3, 3.3), seed=0,
                  device="cuda", stream=None) -> torch.Tensor:
    """fn_params into a new (N, 8) int32 CUDA tensor (fields in PARAMS_DTYPE order)."""
    out = torch.empty((max(N, 0), 8), dtype=torch.int32, device=device)
    fn_params(seed, N, H, W, flip_p, erase_p, scale[0], scale[1], ratio[0], ratio[1], out, stream)
    return out


def params_to_numpy(t: torch.Tensor) -> np.ndarray:
    """(N, 8) int32 tensor -> structured array with PARAMS_DTYPE fields."""
    return np.ascontiguousarray(t.cpu().numpy()).view(PARAMS_DTYPE).reshape(-1)
