"""The flat-layout kernel through the C ABI: outputs whose rows are not a
whole number of 16-byte vectors (widths such as 299, 227 or 28 at one
channel), outputs aligned only to their element size, and the padded layout
at odd widths.  Same oracle and bars as the compact path (page "(11)
FusedNormalization", sections 5 and 12): fp32 within 2e-6, fp16 within one
fp16 ulp and equal to RNE16(oracle) at the preset constants, erased elements
and pad channels +0, guard bands around the output untouched.  Every offset
of the output within a 16-byte vector must give the same bits as the
16-byte aligned output."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from augmentation_amd import synth

from test_gpu_parity import THREADS, check_values, say  # noqa: F401

pytestmark = pytest.mark.gpu

IMAGENET = (synth.WORKLOADS["imagenet_train"].mean, synth.WORKLOADS["imagenet_train"].std)


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    return binding


def run_guarded(b, x, mean, std, flip_p, erase_p, seed, out_dtype, out_off, strides=None,
                first_sample_id=0):
    """One call with the output `out_off` bytes into a buffer filled with
    0xA5; returns the output bytes after checking the guard bands.  With
    `strides` = (row, image, x0 bytes), `x` is the full source and the call
    reads the window that starts x0 bytes into it."""
    if strides is None:
        N, H, W, C = x.shape
    else:
        N, H, W, C = strides[3]
    oc = 4 if out_dtype == 2 else C
    esz = 4 if out_dtype == 0 else 2
    out_bytes = N * H * W * oc * esz
    guard = 4096
    xt = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda()
    buf = torch.full((guard + out_off + out_bytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = buf.data_ptr() + guard + out_off
    if strides is None:
        b.fn_fused_normalize(xt, N, H, W, C, mean, std, flip_p, erase_p, 0.02, 0.33, 0.3, 3.3,
                             seed, out_dtype, dst)
    else:
        b.fn_fused_normalize_ex(xt.data_ptr() + strides[2], strides[0], strides[1], N, H, W, C,
                                mean, std, flip_p, erase_p, 0.02, 0.33, 0.3, 3.3, seed,
                                first_sample_id, out_dtype, dst)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    lo, hi = guard + out_off, guard + out_off + out_bytes
    assert np.all(host[:lo] == 0xA5) and np.all(host[hi:] == 0xA5), "guard band written"
    return host[lo:hi].copy()


def as_values(raw, shape, out_dtype):
    N, H, W, C = shape
    if out_dtype == 0:
        return raw.view(np.float32).reshape(N, H, W, C)
    oc = 4 if out_dtype == 2 else C
    return raw.view(np.float16).reshape(N, H, W, oc)


def check(got, ref, C, out_dtype, what, rne_exact):
    if out_dtype == 2:
        assert np.all(got[..., C:].view(np.uint16) == 0), (what, "pad channels")
        got = np.ascontiguousarray(got[..., :C])
    check_values(got, ref, what, rne_exact=rne_exact)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_every_output_offset_gives_the_aligned_bits(b, out_dtype):
    """A 299-wide batch of several tiles per image (vectors shared by
    neighbouring tiles at every row-tile boundary) with the output at each
    element offset within a 16-byte vector: each offset equals the oracle
    and, bit for bit, the 16-byte aligned output."""
    shape = (3, 40, 299, 3)
    x = np.random.default_rng(11).integers(0, 256, size=shape, dtype=np.uint8)
    mean, std = IMAGENET
    seed = 77
    ref, _ = oracle.fused_normalize(x, mean, std, 1.0 if out_dtype else 0.5, 1.0, seed=seed)
    esz = 4 if out_dtype == 0 else 2
    first = None
    for k in range(16 // esz):
        say(f"flat offsets: out_dtype={out_dtype} offset={k * esz} bytes")
        raw = run_guarded(b, x, mean, std, 1.0 if out_dtype else 0.5, 1.0, seed, out_dtype, k * esz)
        check(as_values(raw, shape, out_dtype), ref, 3, out_dtype, f"offset {k * esz}", True)
        if first is None:
            first = raw
        else:
            assert np.array_equal(raw, first), f"offset {k * esz} differs from the aligned output"


FLAT_SHAPES = [(4, 31, 299, 3), (3, 23, 227, 3), (2, 17, 225, 3), (200, 28, 28, 1),
               (5, 9, 33, 3), (3, 7, 7, 2), (2, 11, 13, 4), (2, 64, 511, 1), (2, 6, 2045, 3),
               (9, 5, 3, 3), (1, 1, 1, 1)]


@pytest.mark.parametrize("shape", FLAT_SHAPES)
@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_widths_that_split_vectors(b, shape, out_dtype):
    """Rows that end inside a 16-byte vector, one or several images per tile,
    rows longer than one pass of the lanes, random constants; the output
    16-byte aligned and 2 or 4 bytes past that."""
    N, H, W, C = shape
    rng = np.random.default_rng(sum(shape) + 31 * out_dtype)
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    mean = tuple(float(v) for v in rng.uniform(0.3, 0.6, C))
    std = tuple(float(v) for v in rng.uniform(0.2, 0.3, C))
    seed = 500 + N * W
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 0.75, seed=seed, threads=THREADS)
    esz = 4 if out_dtype == 0 else 2
    for off in (0, esz, 3 * esz):
        say(f"flat: shape={shape} out_dtype={out_dtype} out_off={off}")
        raw = run_guarded(b, x, mean, std, 0.5, 0.75, seed, out_dtype, off)
        check(as_values(raw, shape, out_dtype), ref, C, out_dtype, f"{shape} off={off}", False)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_crop_windows_of_odd_width(b, out_dtype):
    """fn_fused_normalize_ex windows of odd width from a larger source (row
    and image strides), a nonzero first_sample_id, the output off its
    16-byte alignment: equal to the oracle on the window copied out."""
    src = np.random.default_rng(5).integers(0, 256, size=(6, 64, 80, 3), dtype=np.uint8)
    y0, x0, H, W = 5, 7, 50, 61
    win = np.ascontiguousarray(src[:, y0:y0 + H, x0:x0 + W, :])
    mean, std = IMAGENET
    seed, first = 21, 1000
    ref, _ = oracle.fused_normalize(win, mean, std, 0.5, 1.0, seed=seed, first_n=first)
    say(f"flat crop: out_dtype={out_dtype}")
    raw = run_guarded(b, src, mean, std, 0.5, 1.0, seed, out_dtype, 3 * (4 if out_dtype == 0 else 2),
                      strides=(80 * 3, 64 * 80 * 3, (y0 * 80 + x0) * 3, (6, H, W, 3)),
                      first_sample_id=first)
    check(as_values(raw, (6, H, W, 3), out_dtype), ref, 3, out_dtype, "crop", True)


def test_inception_sized_batch(b):
    """64 images of 299x299x3 -> fp16 at the ImageNet constants, flip and
    erase 0.5: every element equals RNE16(oracle)."""
    shape = (64, 299, 299, 3)
    x = np.random.default_rng(299).integers(0, 256, size=shape, dtype=np.uint8)
    mean, std = IMAGENET
    say("flat: inception-sized batch")
    xt = torch.from_numpy(x).cuda()
    out = b.fused_normalize(xt, mean, std, flip_p=0.5, erase_p=0.5, seed=123, out_dtype=1)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 0.5, seed=123, threads=THREADS)
    check_values(out.cpu().numpy(), ref, "299x299", rne_exact=True)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_flat_kernel_gives_the_tiles_kernel_bits(b, out_dtype):
    """224-wide rows: the 16-byte aligned output takes the tiles kernel, the
    same call with the output one, three and five elements past alignment
    takes the flat kernel; all give the same bits, at random constants (the
    two-fma form) and at the ImageNet constants (one fma)."""
    shape = (4, 30, 224, 3)
    x = np.random.default_rng(224).integers(0, 256, size=shape, dtype=np.uint8)
    esz = 4 if out_dtype == 0 else 2
    rng = np.random.default_rng(9)
    for mean, std in (IMAGENET, (tuple(rng.uniform(0.3, 0.6, 3)), tuple(rng.uniform(0.2, 0.3, 3)))):
        mean = tuple(float(v) for v in mean)
        std = tuple(float(v) for v in std)
        aligned = run_guarded(b, x, mean, std, 0.5, 1.0, 31, out_dtype, 0)
        for k in (1, 3, 5):
            say(f"flat vs tiles: out_dtype={out_dtype} offset={k * esz} bytes")
            raw = run_guarded(b, x, mean, std, 0.5, 1.0, 31, out_dtype, k * esz)
            assert np.array_equal(raw, aligned), f"offset {k * esz}: flat kernel bits differ"


def test_flat_kernel_beyond_4gib(b):
    """28,700 images of 224x224x3 (more than 2^32 input bytes, 8.6 GB of fp16
    output) written once 16-byte aligned (tiles kernel) and once 2 bytes past
    that (flat kernel): the two outputs are the same bits over the whole
    batch, and the images on both sides of the 4 GiB input boundary, the
    first and the last equal RNE16(oracle) -- 32-bit offset arithmetic in
    the flat kernel would show here.  The input is drawn on the GPU from a
    seeded generator."""
    N, H, W, C = 28700, 224, 224, 3
    img = H * W * C
    assert N * img > 2**32
    g = torch.Generator(device="cuda")
    g.manual_seed(4243)
    say(f"flat beyond 4 GiB: {N} images")
    x = torch.randint(0, 256, (N, H, W, C), dtype=torch.uint8, device="cuda", generator=g)
    mean, std = IMAGENET
    args = (N, H, W, C, mean, std, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 777, 1)
    aligned = torch.empty((N, H, W, C), dtype=torch.float16, device="cuda")
    b.fn_fused_normalize(x, *args, aligned)
    buf = torch.empty(N * img * 2 + 16, dtype=torch.uint8, device="cuda")
    b.fn_fused_normalize(x, *args, buf.data_ptr() + 2)
    torch.cuda.synchronize()
    shifted = buf[2:2 + N * img * 2].view(torch.int16).view(N, H, W, C)
    same = all(torch.equal(aligned[i:i + 2048].view(torch.int16), shifted[i:i + 2048])
               for i in range(0, N, 2048))
    assert same, "flat kernel bits differ from the tiles kernel's"
    boundary = 2**32 // img
    picks = [0, boundary - 1, boundary, boundary + 1, N - 1]
    idx = torch.tensor(picks, device="cuda")
    xs = x.index_select(0, idx).cpu().numpy()
    got = shifted.index_select(0, idx).cpu().numpy().view(np.float16)
    del x, aligned, buf, shifted
    torch.cuda.empty_cache()
    for k, n in enumerate(picks):
        ref, _ = oracle.fused_normalize(xs[k:k + 1], mean, std, 0.5, 0.5, seed=777, first_n=n)
        check_values(got[k:k + 1], ref, f"flat beyond 4 GiB, image {n}")


def test_flat_kernel_graph_capture_replays_match_eager(b):
    """The flat kernel, like the tiles kernel, allocates nothing and issues
    no memset: a captured call (299-wide rows, fp16) replayed five times,
    with eager work between replays, each equal to the eager call."""
    shape = (64, 40, 299, 3)
    N, H, W, C = shape
    xt = torch.from_numpy(np.random.default_rng(31).integers(0, 256, size=shape, dtype=np.uint8)).cuda()
    mean, std = IMAGENET
    args = (N, H, W, C, mean, std, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 55, 1)
    eager = torch.empty(shape, dtype=torch.float16, device="cuda")
    b.fn_fused_normalize(xt, *args, eager)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        b.fn_fused_normalize(xt, *args, out, s)
    torch.cuda.synchronize()
    for k in range(5):
        say(f"flat graph replay {k}")
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), k
        _ = (xt.float() * 2).sum().item()  # unrelated eager work between replays


# Rows wider than the usual tiles, each shape aimed at one route through the
# library (comments: the kernel the host picks on a device with 160 KB of LDS
# per work-group and per compute unit).
WIDE = [
    ((1, 3, 12000, 3), 1, 0),   # one-row tiles of 36 KB: tiles kernel
    ((1, 3, 12001, 3), 1, 2),   # one-row tiles, rows inside vectors: flat kernel
    ((1, 2, 28000, 3), 1, 0),   # 84 KB rows, W a multiple of 16, aligned: pixel-group kernel
    ((1, 2, 28000, 3), 1, 2),   # the same rows, output off alignment: flat, one work-group per CU
    ((1, 2, 28001, 3), 0, 0),   # 84 KB rows, odd width, fp32: flat, one work-group per CU
    ((1, 2, 28001, 3), 2, 0),   # the same, padded layout
    ((1, 2, 56000, 3), 1, 0),   # 168 KB rows (beyond LDS), aligned: pixel-group kernel
    ((1, 2, 56001, 3), 1, 0),   # 168 KB rows, odd width: element-wise kernel
]


@pytest.mark.parametrize("case", WIDE)
def test_wide_rows(b, case):
    shape, out_dtype, out_off = case
    N, H, W, C = shape
    x = np.random.default_rng(W).integers(0, 256, size=shape, dtype=np.uint8)
    mean, std = IMAGENET
    seed = 600 + W
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 1.0, seed=seed)
    say(f"wide rows: {shape} out_dtype={out_dtype} out_off={out_off}")
    raw = run_guarded(b, x, mean, std, 0.5, 1.0, seed, out_dtype, out_off)
    check(as_values(raw, shape, out_dtype), ref, C, out_dtype, f"wide {shape}", True)


def test_wide_strided_window(b):
    """A 30,000-pixel window (90 KB rows) read through row and image strides
    (one-row tiles with strided loads), odd offset into the source."""
    src = np.random.default_rng(30000).integers(0, 256, size=(2, 3, 30011, 3), dtype=np.uint8)
    y0, x0, H, W = 1, 5, 2, 30000
    win = np.ascontiguousarray(src[:, y0:y0 + H, x0:x0 + W, :])
    mean, std = IMAGENET
    ref, _ = oracle.fused_normalize(win, mean, std, 0.5, 1.0, seed=8, first_n=3)
    say("wide strided window")
    raw = run_guarded(b, src, mean, std, 0.5, 1.0, 8, 1, 0,
                      strides=(30011 * 3, 3 * 30011 * 3, (y0 * 30011 + x0) * 3, (2, H, W, 3)),
                      first_sample_id=3)
    check(as_values(raw, (2, H, W, 3), 1), ref, 3, 1, "wide strided", True)
