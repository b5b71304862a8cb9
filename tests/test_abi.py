"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects invalid arguments with the documented codes
before touching the GPU (no kernel is launched here)."""
from __future__ import annotations

import os
import re
import subprocess

import numpy as np
import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fn.h")


@pytest.fixture(scope="module")
def b():
    from augmentation_amd import binding
    return binding


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(b):
    declared = declared_functions()
    assert set(declared) == set(b.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared), exported ^ set(declared)
    for name in declared:
        assert hasattr(b._lib, name)


def test_timeline_build_exports_the_same_symbols_and_validates(b):
    """The instrumented build libfn_timeline.so (bench.py --timeline) has the
    product's entry points; its fn_test_timeline checks its arguments."""
    import os
    if not os.path.exists(b.TIMELINE_LIB_PATH):
        pytest.skip("libfn_timeline.so is not built")
    out = subprocess.run(["nm", "-D", "--defined-only", b.TIMELINE_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared_functions())
    L = b.timeline_library()
    assert L.fn_test_timeline(None, -1) == -1
    assert L.fn_test_timeline(None, 5) == -1    # NULL buffer for 5 tiles
    assert L.fn_test_timeline(None, 0) == 0     # recording off


def test_params_struct_is_32_bytes(b):
    import oracle
    assert b.PARAMS_DTYPE.itemsize == 32
    assert b.PARAMS_DTYPE == oracle.PARAMS_DTYPE  # the same eight int32 fields, same order


DEFAULT = dict(N=4, H=8, W=8, C=3, mean=(0.5, 0.5, 0.5), std=(0.25, 0.25, 0.25), flip_p=0.5,
               erase_p=0.5, scale_min=0.02, scale_max=0.33, ratio_min=0.3, ratio_max=3.3, seed=1,
               out_dtype=0)


def call_fused(b, **kw):
    a = dict(DEFAULT, **kw)
    C = a["C"]
    mean = (ctypes_floats(a["mean"], C) if a["mean"] is not None else None)
    std = (ctypes_floats(a["std"], C) if a["std"] is not None else None)
    return b._lib.fn_fused_normalize(None, a["N"], a["H"], a["W"], C, mean, std, a["flip_p"],
                                     a["erase_p"], a["scale_min"], a["scale_max"], a["ratio_min"],
                                     a["ratio_max"], a["seed"], a["out_dtype"], None, None)


def ctypes_floats(v, C):
    import ctypes
    arr = (ctypes.c_float * max(C, 1))()
    for k in range(min(C, len(v))):
        arr[k] = v[k]
    return arr


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), -1), (dict(W=-3), -1), (dict(C=0), -1), (dict(C=5), -1), (dict(N=-1), -1),
    (dict(flip_p=1.5), -1), (dict(flip_p=float("nan")), -1), (dict(erase_p=-0.1), -1),
    (dict(scale_min=0.0), -1), (dict(scale_min=0.5, scale_max=0.4), -1), (dict(scale_max=1.5), -1),
    (dict(ratio_min=0.0), -1), (dict(ratio_min=3.0, ratio_max=2.0), -1),
    (dict(ratio_max=2.0**31), -1), (dict(out_dtype=3), -1), (dict(out_dtype=-1), -1),
    (dict(mean=None), -1),
    (dict(std=(0.2, 0.0, 0.2)), -1), (dict(std=(0.2, -1.0, 0.2)), -1),
    (dict(mean=(0.1, float("inf"), 0.1)), -1), (dict(std=(0.2, float("nan"), 0.2)), -1),
    (dict(H=4097, W=4096), -2),
    (dict(N=2**61, H=16, W=16, C=4, mean=(0, 0, 0, 0), std=(1, 1, 1, 1)), -2),
    (dict(N=4), -1),  # NULL in/out with N > 0
])
def test_invalid_arguments_rejected(b, kw, code):
    rc = call_fused(b, **kw)
    assert rc == code
    assert b.fn_last_error() != ""


def test_zero_images_is_a_no_op(b):
    assert call_fused(b, N=0) == 0
    assert b.fn_last_error() == ""
    assert b._lib.fn_params(1, 0, 8, 8, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, None, None) == 0


def test_scalar_domain_edges_accepted(b):
    for kw in (dict(flip_p=0.0, erase_p=0.0), dict(flip_p=1.0, erase_p=1.0),
               dict(scale_min=2.0**-30, scale_max=1.0), dict(ratio_min=2.0**-30, ratio_max=2.0**30),
               dict(H=4096, W=4096, C=1), dict(C=4, mean=(0, 0, 0, 0), std=(1, 1, 1, 1)),
               dict(out_dtype=2), dict(out_dtype=2, C=1, mean=(0.5,), std=(0.25,))):
        assert call_fused(b, N=0, **kw) == 0, (kw, b.fn_last_error())


def test_params_and_hooks_validate(b):
    L = b._lib
    assert L.fn_params(1, -1, 8, 8, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, None, None) == -1
    assert L.fn_params(1, 4, 8, 8, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, None, None) == -1  # NULL out
    assert L.fn_test_cr_ops(3, None, None, 1, None, None) == -1
    assert L.fn_test_cr_ops(0, None, None, 0, None, None) == 0
    assert L.fn_test_stream(None, None, 16, 3, None) == -1   # widen must be 2 or 4
    assert L.fn_test_stream(None, None, 24, 2, None) == -1   # a multiple of 16 bytes
    assert L.fn_test_stream(None, None, 0, 4, None) == 0
    assert L.fn_test_stream(None, None, 16, 2, None) == -1   # NULL buffers
    assert L.fn_test_timeline(None, 0) == -1                 # the product build records nothing
    assert "timeline" in b.fn_last_error()
    assert L.fn_test_erase_dims(None, None, 0, 8, 8, 0.02, 0.33, 0.3, 3.3, None, None, None,
                                None) == 0
    assert L.fn_test_erase_dims(None, None, 1, 0, 8, 0.02, 0.33, 0.3, 3.3, None, None, None,
                                None) == -1


def test_error_message_is_per_call(b):
    assert call_fused(b, C=9) == -1
    assert "C must be" in b.fn_last_error()
    assert call_fused(b, N=0) == 0
    assert b.fn_last_error() == ""


def test_product_path_does_not_touch_the_oracle():
    """The HIP library and its binding neither import, include nor link the
    oracle; the oracle imports nothing from the product path."""
    pkg = os.path.join(ROOT, "augmentation_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f
    otext = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert "fn_" not in re.sub(r"/\*.*?\*/", "", otext, flags=re.S)
    otext = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert not re.search(r"^\s*(from|import)\s+augmentation_amd", otext, flags=re.M)


def call_fused_ex(b, row_stride, image_stride, first_sample_id, **kw):
    a = dict(DEFAULT, **kw)
    C = a["C"]
    return b._lib.fn_fused_normalize_ex(
        None, row_stride, image_stride, a["N"], a["H"], a["W"], C, ctypes_floats(a["mean"], C),
        ctypes_floats(a["std"], C), a["flip_p"], a["erase_p"], a["scale_min"], a["scale_max"],
        a["ratio_min"], a["ratio_max"], a["seed"], first_sample_id, a["out_dtype"], None, None)


@pytest.mark.parametrize("row_stride,image_stride,first,code", [
    (23, 8 * 24, 0, -1),            # row stride below W*C = 24
    (24, -1, 0, -1),                # negative image stride
    (24, 8 * 24, -5, -1),           # negative first sample
    (2**61, 0, 0, -2),              # (H-1) row strides overflow the span limit
    (24, 2**61, 0, -2),             # (N-1) image strides overflow the span limit
])
def test_ex_invalid_strides_rejected(b, row_stride, image_stride, first, code):
    assert call_fused_ex(b, row_stride, image_stride, first) == code
    assert b.fn_last_error() != ""


def test_ex_valid_layouts_accepted_without_launch(b):
    for rs, ims, first in ((24, 8 * 24, 0), (100, 0, 0), (24, 8 * 24 + 3, 2**40), (31, 1000, 7)):
        assert call_fused_ex(b, rs, ims, first, N=0) == 0, b.fn_last_error()
    assert b._lib.fn_params_ex(1, -1, 4, 8, 8, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, None, None) == -1
    assert b._lib.fn_params_ex(1, 5, 0, 8, 8, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, None, None) == 0
