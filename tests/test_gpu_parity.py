"""GPU parity: the HIP library against the oracle, through the C ABI.

Bars (checked element by element on the same seeded inputs):
  - sample decisions (flip, erase, i, j, eh, ew, attempt, words_used):
    bit-exact;
  - fp32 output: |gpu - oracle| <= 2e-6, erased elements exactly +0.0;
  - fp16 output: |gpu - oracle| <= one fp16 ulp at |oracle|, erased elements
    exactly +0, for any constants.  The kernels carry 1/(255 std) and
    mean/std as fp32 high/low pairs, so their fp32 value is within about one
    fp32 ulp of the oracle's relative to the value itself, also near zero
    where the value cancels.  With the MNIST, CIFAR and ImageNet presets
    every fp16 output also equals the oracle rounded to nearest even (an
    exhaustive check of all 256 byte values per channel shows the kernels'
    fp32 value never crosses an fp16 rounding midpoint there), so preset
    workloads assert that exactly.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from augmentation_amd import synth

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)
FP32_TOL = 2e-6


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    return binding


def say(*a):
    print(*a, flush=True)


def ulp16(ref: np.ndarray) -> np.ndarray:
    """fp16 spacing at |ref| (subnormal spacing below 2^-14)."""
    a = np.maximum(np.abs(ref.astype(np.float64)), 2.0**-14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def erased_mask(P: np.ndarray, H: int, W: int) -> np.ndarray:
    """(N, H, W, 1) bool: pixels inside each sample's erase rectangle."""
    h = np.arange(H)[None, :, None]
    w = np.arange(W)[None, None, :]
    e = P["erase"][:, None, None].astype(bool)
    i, j = P["i"][:, None, None], P["j"][:, None, None]
    eh, ew = P["eh"][:, None, None], P["ew"][:, None, None]
    return (e & (h >= i) & (h < i + eh) & (w >= j) & (w < j + ew))[..., None]


def check_values(got: np.ndarray, ref: np.ndarray, what: str, rne_exact: bool = True,
                 erased: np.ndarray | None = None) -> dict:
    """Compare a GPU output (fp32 or fp16) with the oracle's fp32 result.
    rne_exact: fp16 must equal RNE16(oracle) everywhere (preset constants).
    erased: elements that must be exactly +0; by default the elements where
    the oracle is +0 (no normalized value is exactly 0 at the preset
    constants, so there the two coincide).
    Bounds: fp32 within FP32_TOL of the oracle; fp16 within one fp16 ulp
    at |oracle| of the oracle."""
    assert got.shape == ref.shape, what
    zero = ref.view(np.uint32) == 0 if erased is None else np.broadcast_to(erased, ref.shape)
    if got.dtype == np.float32:
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert float(err.max(initial=0.0)) <= FP32_TOL, (what, float(err.max()))
        assert np.all(got.view(np.uint32)[zero] == 0), what
        return {"max_abs": float(err.max(initial=0.0))}
    assert got.dtype == np.float16
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    u = ulp16(ref)
    bad = err > u
    assert not np.any(bad), (what, int(bad.sum()), float(err.max()))
    assert np.all(got.view(np.uint16)[zero] == 0), what
    same = float(np.mean(got.view(np.uint16) == ref.astype(np.float16).view(np.uint16)))
    if rne_exact:
        assert same == 1.0, (what, same)
    return {"max_abs": float(err.max(initial=0.0)), "rne_equal": same}


def run_fused(b, xt, N, H, W, C, w_or_kw, seed, out_dtype, out=None, stream=None):
    w = w_or_kw
    tdt = torch.float32 if out_dtype == 0 else torch.float16
    if out is None:
        out = torch.empty((N, H, W, C), dtype=tdt, device="cuda")
    b.fn_fused_normalize(xt, N, H, W, C, w["mean"], w["std"], w["flip_p"], w["erase_p"],
                         w["scale"][0], w["scale"][1], w["ratio"][0], w["ratio"][1], seed,
                         out_dtype, out, stream)
    return out


def wl_dict(w: synth.Workload) -> dict:
    return dict(mean=w.mean, std=w.std, flip_p=w.flip_p, erase_p=w.erase_p, scale=w.scale,
                ratio=w.ratio)


def gpu_params(b, w: synth.Workload, seed: int) -> np.ndarray:
    t = b.sample_params(w.N, w.H, w.W, w.flip_p, w.erase_p, w.scale, w.ratio, seed)
    torch.cuda.synchronize()
    return b.params_to_numpy(t)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_params_bit_exact(b, name):
    w = synth.WORKLOADS[name]
    for seed in w.seeds:
        say(f"params: {name} N={w.N} {w.H}x{w.W} seed={seed}")
        got = gpu_params(b, w, seed)
        ref = oracle.params(seed, 0, w.N, w.H, w.W, w.flip_p, w.erase_p, w.scale, w.ratio)
        rows = np.flatnonzero(np.any(got.view(np.int32).reshape(-1, 8) !=
                                     ref.view(np.int32).reshape(-1, 8), axis=1))
        assert rows.size == 0, (name, seed, rows.size, rows[:5], got[rows[:3]], ref[rows[:3]])


@pytest.mark.parametrize("name", ["mnist", "cifar", "imagenet_train", "imagenet_val"])
def test_fused_full_batch(b, name):
    w = synth.WORKLOADS[name]
    x = w.make_input()
    seed = w.seeds[0]
    say(f"fused: {name} {x.shape} out_dtype={w.out_dtype} seed={seed}")
    xt = torch.from_numpy(x).cuda()
    out = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), seed, w.out_dtype)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                    seed=seed, threads=THREADS)
    stats = check_values(out.cpu().numpy(), ref, name)
    say(f"  {stats}")
    # the other dtype on the same inputs
    other = 1 - w.out_dtype
    out2 = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), seed, other)
    torch.cuda.synchronize()
    check_values(out2.cpu().numpy(), ref, name + " other dtype")


def test_stress_eight_back_to_back_launches(b):
    """2048 images, eight launches on one stream with seeds 123..130 into
    eight distinct outputs; every launch's decisions and every output
    element are checked, launch by launch in chunks of 256 images to bound
    host memory.  The ImageNet preset makes every fp16 output equal to the
    oracle rounded to nearest even, erased elements included (+0)."""
    w = synth.WORKLOADS["stress"]
    x = w.make_input()
    xt = torch.from_numpy(x).cuda()
    say(f"stress: {x.shape} x{w.launches} launches")
    outs = [torch.empty((w.N, w.H, w.W, w.C), dtype=torch.float16, device="cuda")
            for _ in w.seeds]
    for seed, out in zip(w.seeds, outs):
        run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), seed, w.out_dtype, out)
    torch.cuda.synchronize()
    chunk = 256
    for seed, out in zip(w.seeds, outs):
        P = oracle.params(seed, 0, w.N, w.H, w.W, w.flip_p, w.erase_p, w.scale, w.ratio)
        got_p = gpu_params(b, w, seed)
        assert got_p.tobytes() == P.tobytes(), seed
        for c0 in range(0, w.N, chunk):
            c1 = min(w.N, c0 + chunk)
            ref, _ = oracle.fused_normalize(x[c0:c1], w.mean, w.std, w.flip_p, w.erase_p,
                                            w.scale, w.ratio, seed=seed, first_n=c0,
                                            threads=THREADS)
            got = out[c0:c1].cpu().numpy()
            if not np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16)):
                check_values(got, ref, f"stress seed={seed} images {c0}..{c1 - 1}")
                raise AssertionError(f"stress seed={seed} images {c0}..{c1 - 1}: not RNE16(oracle)")
        say(f"  seed {seed}: {int(P['flip'].sum())} flipped, {int(P['erase'].sum())} erased, "
            f"all {w.N} images equal RNE16(oracle)")
        del out


EDGE_SHAPES = [(3, 5, 7, 1), (2, 9, 5, 2), (4, 6, 5, 3), (2, 3, 3, 4), (1, 1, 1, 3),
               (1, 1, 17, 3), (5, 17, 1, 3), (3, 2, 2, 1), (2, 31, 33, 3), (7, 13, 11, 4),
               (2, 4, 8192, 1), (1, 600, 6, 3), (9, 28, 28, 1), (64, 32, 32, 3),
               (2, 3, 1024, 3), (2, 5, 700, 4), (40, 8, 8, 2), (3, 64, 48, 3),
               # wide rows (27 KB) in one-row tiles; the input offsets below keep
               # the pixel-group kernel out, so every shape takes the tiles
               # kernel or, when a row ends inside a 16-byte vector or the
               # output is only element aligned, the flat one (the wide-row
               # routes are in test_gpu_flat.py)
               (1, 3, 9000, 3), (1, 2, 9001, 3)]


@pytest.mark.parametrize("shape", EDGE_SHAPES)
@pytest.mark.parametrize("out_dtype", [0, 1])
@pytest.mark.parametrize("out_aligned", [True, False])
def test_edge_shapes_with_guards(b, shape, out_dtype, out_aligned):
    """Odd shapes, the input at a byte offset in 1..7, the output either
    16-byte aligned or only element aligned; guard bands around the output
    must stay untouched."""
    N, H, W, C = shape
    rng = np.random.default_rng(sum(shape) + out_dtype)
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    mean = tuple(float(v) for v in rng.uniform(0.3, 0.6, C))
    std = tuple(float(v) for v in rng.uniform(0.2, 0.3, C))
    kw = dict(mean=mean, std=std, flip_p=0.5, erase_p=1.0, scale=(0.02, 0.33), ratio=(0.3, 3.3))
    elems = N * H * W * C
    esz = 4 if out_dtype == 0 else 2
    in_off = 1 + (sum(shape) % 7)          # input at a byte offset in 1..7
    out_off = 4096 if out_aligned else 4096 + esz
    guard = 4096
    say(f"edge: shape={shape} out_dtype={out_dtype} in_off={in_off} out_off={out_off}")
    in_buf = torch.zeros(elems + in_off + 64, dtype=torch.uint8, device="cuda")
    in_buf[in_off:in_off + elems] = torch.from_numpy(x.reshape(-1)).cuda()
    out_buf = torch.full((out_off + elems * esz + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    seed = 1000 + N + out_off
    b.fn_fused_normalize(in_buf.data_ptr() + in_off, N, H, W, C, mean, std, kw["flip_p"],
                         kw["erase_p"], 0.02, 0.33, 0.3, 3.3, seed, out_dtype,
                         out_buf.data_ptr() + out_off)
    torch.cuda.synchronize()
    host = out_buf.cpu().numpy()
    assert np.all(host[:out_off] == 0xA5) and np.all(host[out_off + elems * esz:] == 0xA5)
    got = host[out_off:out_off + elems * esz].view(np.float32 if out_dtype == 0 else np.float16)
    ref, _ = oracle.fused_normalize(x, mean, std, kw["flip_p"], kw["erase_p"], seed=seed)
    check_values(got.reshape(shape), ref, str(shape), rne_exact=False)


def test_largest_image(b):
    """H*W = 2^24, the largest image the sampler's exact area allows."""
    N, H, W, C = 1, 4096, 4096, 3
    x = np.random.default_rng(5).integers(0, 256, size=(N, H, W, C), dtype=np.uint8)
    say(f"largest: {x.shape}")
    xt = torch.from_numpy(x).cuda()
    kw = dict(mean=synth.IMAGENET_MEAN, std=synth.IMAGENET_STD, flip_p=1.0, erase_p=1.0,
              scale=synth.ERASE_SCALE, ratio=synth.ERASE_RATIO)
    out = run_fused(b, xt, N, H, W, C, kw, 77, 1)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_normalize(x, kw["mean"], kw["std"], 1.0, 1.0, seed=77, threads=THREADS)
    check_values(out.cpu().numpy(), ref, "4096x4096x3")


def test_zero_images_writes_nothing(b):
    out = torch.full((64,), 7.0, device="cuda")
    b.fn_fused_normalize(0, 0, 8, 8, 3, (0.5,) * 3, (0.25,) * 3, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 1,
                         0, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_result_independent_of_batch_size_and_repeatable(b):
    w = synth.WORKLOADS["cifar"]
    x = w.make_input()
    xt = torch.from_numpy(x).cuda()
    full = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 5, 0)
    again = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 5, 0)
    head = run_fused(b, xt[:10].contiguous(), 10, w.H, w.W, w.C, wl_dict(w), 5, 0)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int32), again.view(torch.int32))
    assert torch.equal(full[:10].view(torch.int32), head.view(torch.int32))


def test_page_fp32_vs_fp16_consistency(b):
    """Page "(11)" section 13: 28x28 grey batch, fp32 and fp16 outputs agree
    to MSE < 1e-5 and max relative error < 1e-3 over |v| > 1e-6."""
    w = synth.WORKLOADS["mnist"]
    xt = torch.from_numpy(w.make_input()).cuda()
    o32 = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 123, 0).cpu().numpy().astype(np.float64)
    o16 = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 123, 1).cpu().numpy().astype(np.float64)
    keep = np.abs(o32) > 1e-6
    assert np.mean((o32 - o16) ** 2) < 1e-5
    assert np.max(np.abs(o32[keep] - o16[keep]) / np.abs(o32[keep])) < 1e-3


@pytest.mark.parametrize("ratio", [(0.3, 3.3), (0.5, 4.0), (1.0, 1.0), (2.0**-30, 2.0**30)])
def test_erase_attempts_exhaustive_over_ratio_words(b, ratio):
    """Every one of the 2^24 log-ratio draws (random area words): sides and
    acceptance bit-exact against the oracle."""
    n = 2**24
    rng = np.random.default_rng(len(str(ratio)))
    w_ratio = (np.arange(n, dtype=np.uint64) << np.uint64(8) | rng.integers(0, 256, n, dtype=np.uint64)).astype(np.uint32)
    w_scale = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    H, W = 224, 224
    say(f"erase dims: ratio={ratio}")
    ws, wr = torch.from_numpy(w_scale).cuda(), torch.from_numpy(w_ratio).cuda()
    eh = torch.empty(n, dtype=torch.int32, device="cuda")
    ew = torch.empty(n, dtype=torch.int32, device="cuda")
    acc = torch.empty(n, dtype=torch.uint8, device="cuda")
    b.fn_test_erase_dims(ws, wr, n, H, W, 0.02, 0.33, ratio[0], ratio[1], eh, ew, acc)
    torch.cuda.synchronize()
    r_eh, r_ew, r_acc = oracle.erase_dims_array(w_scale, w_ratio, H, W, (0.02, 0.33), ratio)
    np.testing.assert_array_equal(eh.cpu().numpy(), r_eh)
    np.testing.assert_array_equal(ew.cpu().numpy(), r_ew)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(bool), r_acc)


def test_correctly_rounded_ops(b):
    rng = np.random.default_rng(8)
    # exp: a strided sweep over every binade of 2^-30 <= |L| <= 46, both signs
    bits = np.arange(0x30800000, 0x42380000, 31, dtype=np.uint32)
    L = np.concatenate([bits, bits | np.uint32(0x80000000)]).view(np.float32)
    # sqrt: strided sweep over all positive normal floats
    sq = np.arange(0x00800000, 0x7F800000, 101, dtype=np.uint32).view(np.float32)
    # division: random positive normal pairs with a normal quotient
    a = rng.integers(0x00800000, 0x7F800000, 10_000_000, dtype=np.uint32).view(np.float32)
    d = rng.integers(0x00800000, 0x7F800000, 10_000_000, dtype=np.uint32).view(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        q = a / d
    keep = (q >= np.float32(2.0**-126)) & np.isfinite(q)
    a, d, q = a[keep], d[keep], q[keep]
    for op, x, y, ref in ((0, L, None, oracle.expf_array(L)), (1, sq, None, np.sqrt(sq)),
                          (2, a, d, q)):
        say(f"cr op {op}: {x.size} values")
        xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        yt = torch.from_numpy(np.ascontiguousarray(y)).cuda() if y is not None else None
        out = torch.empty_like(xt)
        b.fn_test_cr_ops(op, xt, yt, x.size, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, (op, x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_bad_pointers_rejected_without_launch(b):
    x = torch.zeros(2 * 8 * 8 * 3, dtype=torch.uint8, device="cuda")
    out = torch.zeros(2 * 8 * 8 * 3, dtype=torch.float32, device="cuda")
    host = np.zeros(2 * 8 * 8 * 3 * 4, np.uint8)
    args = ((0.5,) * 3, (0.25,) * 3, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 1, 0)
    # an allocation of exactly 1000 bytes, straight from the HIP runtime torch uses
    import ctypes
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    raw = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(raw), ctypes.c_size_t(1000)) == 0
    try:
        cases = {
            "host input": (host.ctypes.data, out),
            "host output": (x, host.ctypes.data),
            "output past the end of its allocation": (x, raw.value + 1000 - 64),
            "misaligned fp32 output": (x, out.data_ptr() + 2),
            "overlap": (out.view(torch.uint8), out),
        }
        for what, (src, dst) in cases.items():
            say(f"bad pointer: {what}")
            with pytest.raises(b.FnError) as e:
                b.fn_fused_normalize(src, 2, 8, 8, 3, *args, dst)
            assert e.value.code == b.FN_EINVAL, what
        # the same raw allocation, used within its size, is accepted
        b.fn_fused_normalize(x, 1, 8, 5, 3, *args, raw.value)
        torch.cuda.synchronize()
    finally:
        hip.hipFree(raw)
    # no sticky HIP error is left behind: torch keeps working
    y = (x.float() + 1).sum()
    torch.cuda.synchronize()
    assert float(y) == x.numel()


def stream_reference(src: np.ndarray, widen: int) -> np.ndarray:
    """What fn_test_stream writes, from its documented layout: widen 2, the
    input widened in order; widen 4, per block of up to 256 input vectors of
    16 bytes, dword k of every vector (its 4 bytes, each zero-extended) forms
    the block's k-th run of output vectors."""
    if widen == 2:
        return src.astype(np.uint16)
    vec = src.reshape(-1, 16)
    out = []
    for b in range(0, len(vec), 256):
        blk = vec[b:b + 256]
        parts = blk.reshape(len(blk), 4, 4).astype(np.uint32)
        out.append(parts.transpose(1, 0, 2).reshape(-1))
    return np.concatenate(out)


@pytest.mark.parametrize("widen", [2, 4])
def test_stream_hook(b, widen):
    """fn_test_stream writes every input byte zero-extended to `widen` bytes,
    in its documented block layout, including a partial last block, and
    nothing beyond its output."""
    n = (1 << 20) + 16 * 37
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.full((n * widen + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    b.fn_test_stream(src, dst, n, widen)
    torch.cuda.synchronize()
    host = dst.cpu().numpy()
    assert np.all(host[n * widen:] == 0xA5)
    got = host[:n * widen].view(np.uint16 if widen == 2 else np.uint32)
    np.testing.assert_array_equal(got, stream_reference(src.cpu().numpy(), widen))


# Constants whose single-fma result is not always the correctly rounded one:
# mean 0.4 puts x = 102 within 3e-8 of an exact cancellation, where one fma on
# rounded constants errs by several fp16 ulps of the tiny result.
CANCELLING = [((0.4, 0.4, 0.4), (0.2, 0.2, 0.2)), ((0.6, 0.2, 0.8), (0.3, 0.7, 0.05)),
              ((1.0, 0.0, 0.5), (1.0, 1.0, 0.5))]


@pytest.mark.parametrize("consts", CANCELLING)
@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_tiles_kernel_with_cancelling_constants(b, consts, out_dtype):
    """The tiles kernel (16-byte aligned output, whole 16-byte vectors per
    row) with constants where values cancel to (near) zero: fp32 within 2e-6,
    fp16 within one fp16 ulp of the oracle, for every byte value."""
    mean, std = consts
    N, H, W, C = 6, 40, 48, 3
    x = np.tile(np.arange(256, dtype=np.uint8), N * H * W * C // 256 + 1)[:N * H * W * C]
    x = np.random.default_rng(3).permutation(x).reshape(N, H, W, C)
    say(f"cancelling constants {consts} out_dtype={out_dtype}")
    xt = torch.from_numpy(x).cuda()
    out = b.fused_normalize(xt, mean, std, 0.5, 0.5, seed=17, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 0.5, seed=17)
    P = oracle.params(17, 0, N, H, W, 0.5, 0.5)
    got = out.cpu().numpy()
    if out_dtype == 2:
        assert np.all(got[..., C:].view(np.uint16) == 0)
        got = np.ascontiguousarray(got[..., :C])
    check_values(got, ref, str(consts), rne_exact=False, erased=erased_mask(P, H, W))


def test_batch_beyond_4gib(b):
    """An input of more than 2^32 bytes (28,700 images of 224x224x3, fp16
    output 8.6 GB): every decision checked, and the images on both sides of
    the 4 GiB input boundary, the first and the last element by element --
    32-bit offset arithmetic anywhere would show here.  The input is drawn
    on the GPU from a seeded generator; sampled images are copied back."""
    N, H, W, C = 28700, 224, 224, 3
    img = H * W * C
    assert N * img > 2**32
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    say(f"beyond 4 GiB: {N} images, {N * img / 2**30:.2f} GiB input")
    x = torch.randint(0, 256, (N, H, W, C), dtype=torch.uint8, device="cuda", generator=g)
    out = torch.empty((N, H, W, C), dtype=torch.float16, device="cuda")
    kw = dict(mean=synth.IMAGENET_MEAN, std=synth.IMAGENET_STD, flip_p=0.5, erase_p=0.5,
              scale=synth.ERASE_SCALE, ratio=synth.ERASE_RATIO)
    run_fused(b, x, N, H, W, C, kw, 999, 1, out)
    t = b.sample_params(N, H, W, 0.5, 0.5, synth.ERASE_SCALE, synth.ERASE_RATIO, 999)
    torch.cuda.synchronize()
    P = oracle.params(999, 0, N, H, W, 0.5, 0.5, synth.ERASE_SCALE, synth.ERASE_RATIO)
    assert b.params_to_numpy(t).tobytes() == P.tobytes()
    boundary = 2**32 // img
    picks = [0, boundary - 1, boundary, boundary + 1, N - 1]
    idx = torch.tensor(picks, device="cuda")
    xs = x.index_select(0, idx).cpu().numpy()
    got = out.index_select(0, idx).cpu().numpy()
    del x, out
    torch.cuda.empty_cache()
    for k, n in enumerate(picks):
        ref, _ = oracle.fused_normalize(xs[k:k + 1], kw["mean"], kw["std"], 0.5, 0.5,
                                        seed=999, first_n=n)
        check_values(got[k:k + 1], ref, f"beyond 4 GiB, image {n}")


def test_graph_capture_replays_match_eager(b):
    """The call allocates nothing and issues no memset, so it can be captured
    in a HIP graph: five replays, with eager work and synchronisations
    between them, each equal to the eager result bit for bit."""
    w = synth.WORKLOADS["cifar"]
    xt = torch.from_numpy(w.make_input()).cuda()
    eager = run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 11, 1)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run_fused(b, xt, w.N, w.H, w.W, w.C, wl_dict(w), 11, 1, out, stream=s)
    torch.cuda.synchronize()
    for k in range(5):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), k
        _ = (xt.float() * 2).sum().item()  # unrelated eager work between replays


def test_concurrent_calls_on_two_streams(b):
    """The library keeps no per-call state on the device: two calls with
    different seeds and output types, enqueued on two streams and free to
    overlap, each equal their own serial result."""
    w = synth.WORKLOADS["imagenet_train"]
    xt = torch.from_numpy(w.make_input()[:128]).cuda()
    N = xt.shape[0]
    ref16 = run_fused(b, xt, N, w.H, w.W, w.C, wl_dict(w), 5, 1)
    ref32 = run_fused(b, xt, N, w.H, w.W, w.C, wl_dict(w), 6, 0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o16 = torch.empty_like(ref16)
    o32 = torch.empty_like(ref32)
    for _ in range(3):
        o16.fill_(float("nan"))
        o32.fill_(float("nan"))
        torch.cuda.synchronize()
        run_fused(b, xt, N, w.H, w.W, w.C, wl_dict(w), 5, 1, o16, stream=s1)
        run_fused(b, xt, N, w.H, w.W, w.C, wl_dict(w), 6, 0, o32, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(o16.view(torch.int16), ref16.view(torch.int16))
        assert torch.equal(o32.view(torch.int32), ref32.view(torch.int32))


def test_calls_from_several_host_threads(b):
    """The host side is reentrant: four threads, each on its own stream with
    its own constants, output type and seed (so each thread's memo of the
    one-fma check and its error buffer differ), call the library 25 times
    each while the others do; every output equals its serial result, and an
    invalid call in one thread reports its own error there."""
    import threading
    w = synth.WORKLOADS["imagenet_train"]
    xt = torch.from_numpy(w.make_input()[:32]).cuda()
    N = xt.shape[0]
    jobs = [((0.485, 0.456, 0.406), (0.229, 0.224, 0.225), 1, 11),
            ((0.4, 0.4, 0.4), (0.2, 0.2, 0.2), 0, 12),
            ((0.5, 0.5, 0.5), (0.25, 0.25, 0.25), 2, 13),
            ((0.3, 0.6, 0.1), (0.3, 0.17, 0.45), 1, 14)]
    refs = []
    for mean, std, od, seed in jobs:
        refs.append(b.fused_normalize(xt, mean, std, 0.5, 0.5, (0.02, 0.33), (0.3, 3.3), seed, od))
    torch.cuda.synchronize()
    errors = []

    def worker(j):
        mean, std, od, seed = jobs[j]
        s = torch.cuda.Stream()
        out = torch.empty_like(refs[j])
        try:
            for it in range(25):
                b.fused_normalize(xt, mean, std, 0.5, 0.5, (0.02, 0.33), (0.3, 3.3), seed, od,
                                  out=out, stream=s)
                if it % 5 == 0:
                    try:  # flip_p = 2: rejected by the library before any launch
                        b.fn_fused_normalize(xt, N, w.H, w.W, w.C, mean, std, 2.0, 0.5, 0.02,
                                             0.33, 0.3, 3.3, seed, od, out, s)
                        errors.append((j, "invalid call accepted"))
                    except b.FnError as e:
                        if "flip_p must be in [0, 1]" not in str(e):
                            errors.append((j, str(e)))
                s.synchronize()
                view = torch.int32 if od == 0 else torch.int16
                if not torch.equal(out.view(view), refs[j].view(view)):
                    errors.append((j, f"iteration {it} differs"))
        except Exception as e:  # noqa: BLE001
            errors.append((j, repr(e)))

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors[:5]
