"""Seeded random cases through the C ABI against the oracle: shapes with 1-4
channels and widths from 1 to about 3,000 pixels, every output type, output
offsets within a 16-byte vector, strided windows of larger sources, random
constants and probabilities, nonzero first_sample_id.  Each case reaches one
of the library's kernels (tiles, flat, or their wide-row and multi-image
forms); guard bands around the output must stay untouched.  Bars as in the
other parity tests (page "(11) FusedNormalization", sections 5 and 12)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

from test_gpu_flat import as_values, check, run_guarded  # noqa: F401
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

CASES = 1000


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    return binding


def make_case(k):
    rng = np.random.default_rng(9000 + k)
    C = int(rng.integers(1, 5))
    W = int(np.exp(rng.uniform(0, np.log(3000))))
    H = int(rng.integers(1, 41))
    N = int(max(1, min(6, 400_000 // max(1, H * W * C))))
    N = int(rng.integers(1, N + 1))
    out_dtype = int(rng.integers(0, 3))
    esz = 4 if out_dtype == 0 else 2
    out_off = esz * int(rng.integers(0, 16 // esz)) if rng.random() < 0.5 else 0
    strided = rng.random() < 0.35
    if rng.random() < 0.5:
        mean = tuple(float(v) for v in rng.uniform(0.0, 1.0, C))
        # std >= 0.13 keeps |value| below 8, where the fp32 bar of 2e-6 holds
        std = tuple(float(v) for v in rng.uniform(0.13, 0.5, C))
    else:
        mean, std = (0.5,) * C, (0.25,) * C
    flip_p = float(rng.choice([0.0, 0.5, 1.0]))
    erase_p = float(rng.choice([0.0, 0.5, 1.0]))
    seed = int(rng.integers(0, 2**63))
    first = int(rng.integers(0, 2**40)) if rng.random() < 0.3 else 0
    return dict(N=N, H=H, W=W, C=C, out_dtype=out_dtype, out_off=out_off, strided=strided,
                mean=mean, std=std, flip_p=flip_p, erase_p=erase_p, seed=seed, first=first,
                rng=rng)


@pytest.mark.parametrize("k", range(CASES))
def test_random_case(b, k):
    c = make_case(k)
    N, H, W, C = c["N"], c["H"], c["W"], c["C"]
    rng = c["rng"]
    say(f"random case {k}: N={N} H={H} W={W} C={C} out={c['out_dtype']} off={c['out_off']} "
        f"strided={c['strided']} flip={c['flip_p']} erase={c['erase_p']} first={c['first']}")
    if c["strided"]:
        sh, sw = H + int(rng.integers(0, 4)), W + int(rng.integers(0, 9))
        y0, x0 = int(rng.integers(0, sh - H + 1)), int(rng.integers(0, sw - W + 1))
        src = rng.integers(0, 256, size=(N, sh, sw, C), dtype=np.uint8)
        x = np.ascontiguousarray(src[:, y0:y0 + H, x0:x0 + W, :])
        strides = (sw * C, sh * sw * C, (y0 * sw + x0) * C, (N, H, W, C))
        raw = run_guarded(b, src, c["mean"], c["std"], c["flip_p"], c["erase_p"], c["seed"],
                          c["out_dtype"], c["out_off"], strides=strides, first_sample_id=c["first"])
    else:
        x = rng.integers(0, 256, size=(N, H, W, C), dtype=np.uint8)
        if c["first"]:
            strides = (W * C, H * W * C, 0, (N, H, W, C))
            raw = run_guarded(b, x, c["mean"], c["std"], c["flip_p"], c["erase_p"], c["seed"],
                              c["out_dtype"], c["out_off"], strides=strides,
                              first_sample_id=c["first"])
        else:
            raw = run_guarded(b, x, c["mean"], c["std"], c["flip_p"], c["erase_p"], c["seed"],
                              c["out_dtype"], c["out_off"])
    ref, _ = oracle.fused_normalize(x, c["mean"], c["std"], c["flip_p"], c["erase_p"],
                                    seed=c["seed"], first_n=c["first"])
    check(as_values(raw, (N, H, W, C), c["out_dtype"]), ref, C, c["out_dtype"], f"case {k}", False)


WIDE_CASES = 100


@pytest.mark.parametrize("k", range(WIDE_CASES))
def test_random_wide_case(b, k):
    """Rows of 3,000 to 40,000 pixels: one-row tiles up to the LDS limit, the
    pixel-group kernel and the element-wise one, with the same random
    offsets, strides and constants."""
    c = make_case(10_000 + k)
    rng = c["rng"]
    c["W"] = int(np.exp(rng.uniform(np.log(3000), np.log(40000))))
    c["H"] = int(rng.integers(1, 5))
    c["N"] = int(rng.integers(1, 4))
    c["strided"] = c["strided"] and c["W"] * c["C"] < 150_000
    k_orig = k
    N, H, W, C = c["N"], c["H"], c["W"], c["C"]
    say(f"random wide case {k_orig}: N={N} H={H} W={W} C={C} out={c['out_dtype']} "
        f"off={c['out_off']} strided={c['strided']}")
    if c["strided"]:
        sw = W + int(rng.integers(0, 9))
        x0 = int(rng.integers(0, sw - W + 1))
        src = rng.integers(0, 256, size=(N, H, sw, C), dtype=np.uint8)
        x = np.ascontiguousarray(src[:, :, x0:x0 + W, :])
        raw = run_guarded(b, src, c["mean"], c["std"], c["flip_p"], c["erase_p"], c["seed"],
                          c["out_dtype"], c["out_off"], strides=(sw * C, H * sw * C, x0 * C, (N, H, W, C)),
                          first_sample_id=c["first"])
    else:
        x = rng.integers(0, 256, size=(N, H, W, C), dtype=np.uint8)
        raw = run_guarded(b, x, c["mean"], c["std"], c["flip_p"], c["erase_p"], c["seed"],
                          c["out_dtype"], c["out_off"], strides=(W * C, H * W * C, 0, (N, H, W, C)),
                          first_sample_id=c["first"])
    ref, _ = oracle.fused_normalize(x, c["mean"], c["std"], c["flip_p"], c["erase_p"],
                                    seed=c["seed"], first_n=c["first"])
    check(as_values(raw, (N, H, W, C), c["out_dtype"]), ref, C, c["out_dtype"], f"wide case {k}", False)
