"""The host SSE4.1/F16C path (libfn_cpu.so: page "(11) FusedNormalization"'s
own method class, sections 5-8 and 12) against the oracle, on the CPU.

Same bars as the GPU path: decisions bit-exact; fp32 within 2e-6 of the
oracle; fp16 within one fp16 ulp at |oracle| for any constants, and equal to
the oracle rounded to nearest even at the MNIST, CIFAR and ImageNet presets;
erased elements and pad channels +0.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from conftest import ROOT

import oracle
from augmentation_amd import synth

FP32_TOL = 2e-6
THREADS = min(8, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def cs():
    from augmentation_amd import cpu_simd
    return cpu_simd


def ulp16(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref.astype(np.float64)), 2.0**-14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def erased_mask(P, H, W):
    h = np.arange(H)[None, :, None]
    w = np.arange(W)[None, None, :]
    e = P["erase"][:, None, None].astype(bool)
    i, j = P["i"][:, None, None], P["j"][:, None, None]
    eh, ew = P["eh"][:, None, None], P["ew"][:, None, None]
    return (e & (h >= i) & (h < i + eh) & (w >= j) & (w < j + ew))[..., None]


def check(got, ref, P, C, out_dtype, rne_exact, what):
    """got: (N, H, W, OC) output; ref: the oracle's (N, H, W, C) fp32."""
    N, H, W, _ = ref.shape
    if out_dtype == 2:
        assert np.all(got[..., C:].view(np.uint16) == 0), what
        got = np.ascontiguousarray(got[..., :C])
    er = np.broadcast_to(erased_mask(P, H, W), ref.shape)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    if out_dtype == 0:
        assert err.max(initial=0.0) <= FP32_TOL, (what, err.max())
        assert np.all(got.view(np.uint32)[er] == 0), what
    else:
        assert not np.any(err > ulp16(ref)), (what, int((err > ulp16(ref)).sum()))
        assert np.all(got.view(np.uint16)[er] == 0), what
        if rne_exact:
            assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16)), what


def test_library_exports_what_the_header_declares(cs):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fn_cpu.h")).read(),
                  flags=re.S)
    declared = set(re.findall(r"\b(fn_cpu_\w+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", cs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert declared == exported == set(cs.EXPORTED)


def test_gpu_library_never_reaches_the_host_path():
    """The GPU binding and library neither import nor link the host path."""
    for f in ("binding.py", "__init__.py"):
        text = open(os.path.join(ROOT, "augmentation_amd", f)).read()
        assert "cpu_simd" not in text and "fn_cpu" not in text, f
    for f in os.listdir(os.path.join(ROOT, "augmentation_amd", "csrc")):
        assert "fn_cpu" not in open(os.path.join(ROOT, "augmentation_amd", "csrc", f)).read(), f


@pytest.mark.parametrize("name", ["mnist", "cifar", "imagenet_train", "imagenet_val"])
def test_workloads_against_the_oracle(cs, name):
    w = synth.WORKLOADS[name]
    x = w.make_input()
    seed = w.seeds[0]
    ref, _ = oracle.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                    seed=seed, threads=THREADS)
    P = oracle.params(seed, 0, w.N, w.H, w.W, w.flip_p, w.erase_p, w.scale, w.ratio)
    for od in (0, 1, 2):
        got, prm = cs.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                      seed=seed, out_dtype=od, threads=THREADS, with_params=True)
        assert prm.tobytes() == P.tobytes(), (name, od)
        check(got, ref, P, w.C, od, True, f"{name} out_dtype={od}")


def test_stress_seeds_decisions_and_first_images(cs):
    """The stress workload's eight seeds: decisions of the first 256 samples
    and those images' outputs."""
    w = synth.WORKLOADS["stress"]
    x = w.make_input()[:256]
    for seed in w.seeds:
        got, prm = cs.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                      seed=seed, out_dtype=1, threads=THREADS, with_params=True)
        P = oracle.params(seed, 0, len(x), w.H, w.W, w.flip_p, w.erase_p, w.scale, w.ratio)
        assert prm.tobytes() == P.tobytes(), seed
        if seed == w.seeds[0]:
            ref, _ = oracle.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale,
                                            w.ratio, seed=seed, threads=THREADS)
            check(got, ref, P, w.C, 1, True, "stress")


SHAPES = [(3, 5, 7, 1), (2, 9, 5, 2), (4, 6, 5, 3), (2, 3, 3, 4), (1, 1, 1, 3), (1, 1, 17, 3),
          (5, 17, 1, 3), (2, 31, 33, 3), (7, 13, 11, 4), (2, 4, 64, 1), (3, 8, 40, 2),
          (4, 16, 29, 3), (2, 5, 6, 4), (2, 3, 1024, 3)]


@pytest.mark.parametrize("shape", SHAPES)
def test_edge_shapes(cs, shape):
    """Odd shapes, every channel count, rows shorter than one 16-byte vector
    and rows with a ragged tail, random constants, erase always tried."""
    N, H, W, C = shape
    rng = np.random.default_rng(sum(shape))
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    mean = rng.uniform(0.3, 0.6, C)
    std = rng.uniform(0.2, 0.3, C)
    seed = 40 + N + W
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 1.0, seed=seed)
    P = oracle.params(seed, 0, N, H, W, 0.5, 1.0)
    for od in (0, 1, 2):
        got = cs.fused_normalize(x, mean, std, 0.5, 1.0, seed=seed, out_dtype=od, threads=3)
        check(got, ref, P, C, od, False, f"{shape} out_dtype={od}")


@pytest.mark.parametrize("consts", [((0.4, 0.4, 0.4), (0.2, 0.2, 0.2)),
                                    ((0.6, 0.2, 0.8), (0.3, 0.7, 0.05))])
def test_cancelling_constants(cs, consts):
    """Constants where the page's fp32 form would miss the fp16 bar near an
    exact cancellation: every byte value, within one fp16 ulp."""
    mean, std = consts
    N, H, W, C = 4, 16, 48, 3
    x = np.random.default_rng(5).permutation(
        np.tile(np.arange(256, dtype=np.uint8), N * H * W * C // 256 + 1)[:N * H * W * C])
    x = x.reshape(N, H, W, C)
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 0.5, seed=9)
    P = oracle.params(9, 0, N, H, W, 0.5, 0.5)
    for od in (0, 1, 2):
        got = cs.fused_normalize(x, mean, std, 0.5, 0.5, seed=9, out_dtype=od, threads=2)
        check(got, ref, P, C, od, False, f"{consts} out_dtype={od}")


def test_slices_reproduce_the_whole_batch(cs):
    w = synth.WORKLOADS["cifar"]
    x = w.make_input()
    whole = cs.fused_normalize(x, w.mean, w.std, 0.5, 0.5, seed=3, out_dtype=1, threads=4)
    cuts = [0, 1, 17, 100, 256]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = cs.fused_normalize(x[a:b], w.mean, w.std, 0.5, 0.5, seed=3, out_dtype=1,
                                  first_sample_id=a, threads=2)
        assert np.array_equal(part.view(np.uint16), whole[a:b].view(np.uint16)), (a, b)
    one = cs.fused_normalize(x, w.mean, w.std, 0.5, 0.5, seed=3, out_dtype=1, threads=1)
    assert np.array_equal(one.view(np.uint16), whole.view(np.uint16))


@pytest.mark.parametrize("kw", [dict(C=5), dict(flip_p=1.5), dict(std=(0.2, 0.0, 0.2)),
                                dict(ratio=(0.0, 3.3)), dict(out_dtype=3), dict(first_sample_id=-1)])
def test_invalid_arguments_rejected(cs, kw):
    C = kw.pop("C", 3)
    args = dict(mean=(0.5,) * C, std=kw.pop("std", (0.25,) * C), flip_p=0.5, erase_p=0.5,
                scale=(0.02, 0.33), ratio=(0.3, 3.3), seed=1, out_dtype=0, first_sample_id=0)
    args.update(kw)
    x = np.zeros((2, 4, 4, C), np.uint8)
    od = args.pop("out_dtype")
    if od not in (0, 1, 2):  # the binding sizes its output by type: call the C entry point
        out = np.zeros((2, 4, 4, C), np.float32)
        m = (ctypes.c_float * C)(*args["mean"])
        s = (ctypes.c_float * C)(*args["std"])
        rc = cs._lib.fn_cpu_fused_normalize(x.ctypes.data, 2, 4, 4, C, m, s, 0.5, 0.5, 0.02, 0.33,
                                            0.3, 3.3, 1, 0, od, out.ctypes.data, None, 1)
        assert rc == -1 and cs._lib.fn_cpu_last_error()
        return
    with pytest.raises(cs.FnCpuError):
        cs.fused_normalize(x, out_dtype=od, **args)


def test_batch_size_overflow_rejected(cs):
    """N*H*W*16 beyond int64 is refused before anything is read or written."""
    m = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    sd = (ctypes.c_float * 3)(0.25, 0.25, 0.25)
    x = np.zeros(16, np.uint8)
    out = np.zeros(16, np.float32)
    rc = cs._lib.fn_cpu_fused_normalize(x.ctypes.data, 1 << 50, 4096, 4096, 3, m, sd, 0.5, 0.5,
                                        0.02, 0.33, 0.3, 3.3, 1, 0, 0, out.ctypes.data, None, 4)
    assert rc == -1 and b"overflow" in cs._lib.fn_cpu_last_error()
    assert not out.any()
