"""fn_fused_normalize_ex and fn_params_ex through the C ABI.

Strided sources (page "(11) FusedNormalization", section 5: execute() takes
an input row stride; section 4: crops run before the fused step): the
output for a window of a larger source must equal the oracle on that window
copied out compactly -- the plain definition of reading a crop.

first_sample_id (section 10: decisions are a function of seed and offset):
slices [a, b) of a batch called with first_sample_id = a must reproduce the
whole batch bit for bit, decisions and pixels, and fn_params_ex must equal
the oracle's decisions for samples first_sample_id + n."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from augmentation_amd import synth

from test_gpu_parity import THREADS, check_values, erased_mask, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    return binding


IM = dict(mean=synth.IMAGENET_MEAN, std=synth.IMAGENET_STD)

# (N, src_h, src_w, C, H, W, y0, x0, row_pad, image_pad): windows of larger
# sources; row/image pads make strides that are not multiples of 16 (the
# first byte of every row then sits at a different offset in its granule)
WINDOWS = [
    (8, 256, 256, 3, 224, 224, 16, 16, 0, 0),      # centre crop of 256x256
    (4, 256, 256, 3, 224, 224, 3, 29, 5, 11),      # odd offset, odd strides
    (6, 40, 50, 3, 32, 32, 4, 9, 7, 0),            # small images: several per tile
    (5, 30, 30, 1, 28, 28, 1, 2, 3, 13),           # one channel
    (3, 20, 21, 4, 17, 20, 2, 1, 0, 1),            # four channels
    (2, 9, 1100, 3, 7, 1024, 1, 37, 9, 3),         # rows wider than a pass of the lanes
    (3, 12, 14, 2, 12, 13, 0, 1, 1, 0),            # odd width
    # narrow rows of many tall images: each row takes a 32-byte LDS slot, so
    # tiles are sized by slots, not by row bytes
    (1024, 4100, 8, 1, 4096, 4, 2, 3, 0, 0),
    (2048, 1030, 12, 1, 1024, 8, 3, 2, 0, 0),
]


def run_window(b, case, out_dtype, out_aligned, first_sample_id=0, image_stride_zero=False):
    N, sh, sw, C, H, W, y0, x0, rpad, ipad = case
    rng = np.random.default_rng(sum(case) + out_dtype)
    src = rng.integers(0, 256, size=(N, sh, sw * C + rpad), dtype=np.uint8)
    row_stride = sw * C + rpad
    image_stride = 0 if image_stride_zero else sh * row_stride + ipad
    total = (N - 1) * image_stride + sh * row_stride
    flat = np.zeros(total + 64, dtype=np.uint8)
    for n in range(N):
        o = n * image_stride
        flat[o:o + sh * row_stride] = src[0 if image_stride_zero else n].reshape(-1)
    base_off = 5  # the source buffer itself at an odd offset
    buf = torch.zeros(flat.size + base_off, dtype=torch.uint8, device="cuda")
    buf[base_off:] = torch.from_numpy(flat).cuda()
    first = base_off + y0 * row_stride + x0 * C
    # the window, copied out compactly: what the oracle reads
    x = np.lib.stride_tricks.as_strided(flat[y0 * row_stride + x0 * C:], shape=(N, H, W * C),
                                        strides=(image_stride, row_stride, 1))
    x = np.ascontiguousarray(x).reshape(N, H, W, C)
    oc = 4 if out_dtype == 2 else C
    esz = 4 if out_dtype == 0 else 2
    out_off = 4096 if out_aligned else 4096 + esz
    out_bytes = N * H * W * oc * esz
    out = torch.full((out_off + out_bytes + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    seed = 31 + N
    b.fn_fused_normalize_ex(buf.data_ptr() + first, row_stride, image_stride, N, H, W, C,
                            IM["mean"][:C] if C <= 3 else (0.4, 0.45, 0.5, 0.55),
                            IM["std"][:C] if C <= 3 else (0.2, 0.25, 0.22, 0.3),
                            0.5, 0.8, 0.02, 0.33, 0.3, 3.3, seed, first_sample_id, out_dtype,
                            out.data_ptr() + out_off)
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    assert np.all(host[:out_off] == 0xA5) and np.all(host[out_off + out_bytes:] == 0xA5)
    got = host[out_off:out_off + out_bytes].view(np.float32 if esz == 4 else np.float16)
    got = got.reshape(N, H, W, oc)
    mean = IM["mean"][:C] if C <= 3 else (0.4, 0.45, 0.5, 0.55)
    std = IM["std"][:C] if C <= 3 else (0.2, 0.25, 0.22, 0.3)
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 0.8, seed=seed, first_n=first_sample_id,
                                    threads=THREADS)
    P = oracle.params(seed, first_sample_id, N, H, W, 0.5, 0.8)
    return got, ref, erased_mask(P, H, W)


@pytest.mark.parametrize("case", WINDOWS)
@pytest.mark.parametrize("out_dtype", [0, 1, 2])
@pytest.mark.parametrize("out_aligned", [True, False])
def test_window_of_strided_source(b, case, out_dtype, out_aligned):
    say(f"window: {case} out_dtype={out_dtype} aligned={out_aligned}")
    got, ref, er = run_window(b, case, out_dtype, out_aligned)
    C = ref.shape[-1]
    if out_dtype == 2:
        check_values(np.ascontiguousarray(got[..., :C]), ref, str(case), rne_exact=False, erased=er)
        assert np.all(got[..., C:].view(np.uint16) == 0)
    else:
        check_values(got, ref, str(case), rne_exact=False, erased=er)


def test_image_stride_zero_reads_one_image_n_times(b):
    got, ref, er = run_window(b, WINDOWS[0], 1, True, image_stride_zero=True)
    check_values(got, ref, "image stride 0", rne_exact=False, erased=er)


def test_window_with_first_sample_id(b):
    got, ref, er = run_window(b, WINDOWS[1], 1, True, first_sample_id=1000)
    check_values(got, ref, "window + first_sample_id", rne_exact=False, erased=er)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_slices_reproduce_the_whole_batch(b, out_dtype):
    """A batch split into uneven slices [a, b), each called with
    first_sample_id = a on its own slice of the input, equals the call on
    the whole batch bit for bit -- what data-parallel ranks would do."""
    w = synth.WORKLOADS["imagenet_train"]
    x = w.make_input()[:64]
    N = x.shape[0]
    xt = torch.from_numpy(x).cuda()
    oc = 4 if out_dtype == 2 else w.C
    tdt = torch.float32 if out_dtype == 0 else torch.float16
    whole = torch.empty((N, w.H, w.W, oc), dtype=tdt, device="cuda")
    parts = torch.empty_like(whole)
    args = (w.mean, w.std, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 77)
    row, img = w.W * w.C, w.H * w.W * w.C
    b.fn_fused_normalize_ex(xt, row, img, N, w.H, w.W, w.C, *args, 0, out_dtype, whole)
    cuts = [0, 1, 7, 30, 31, 64]
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        say(f"slice [{a_}, {b_}) out_dtype={out_dtype}")
        b.fn_fused_normalize_ex(xt[a_:b_], row, img, b_ - a_, w.H, w.W, w.C, *args, a_, out_dtype,
                                parts[a_:b_])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16 if out_dtype else torch.int32),
                       parts.view(torch.int16 if out_dtype else torch.int32))
    # and the plain entry point is the first_sample_id = 0 case
    plain = b.fused_normalize(xt, w.mean, w.std, 0.5, 0.5, (0.02, 0.33), (0.3, 3.3), 77,
                              out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16 if out_dtype else torch.int32),
                       plain.view(torch.int16 if out_dtype else torch.int32))


@pytest.mark.parametrize("C,out_dtype", [(1, 1), (2, 1), (3, 1), (4, 1), (1, 2), (3, 2)])
def test_long_launch_equals_its_short_slices(b, C, out_dtype):
    """An fp16 launch (packed or 4-channel) long enough for the
    non-temporal-store instance of the tiles kernel (at least 320 MiB moved)
    equals the same batch done as slices of at most 128 images (the
    system-scope-store instance), bit for bit."""
    H = W = 224
    oc = 4 if out_dtype == 2 else C
    N = -(-(320 << 20) // (H * W * (C + 2 * oc))) + 3
    say(f"long launch: N={N} C={C} out_dtype={out_dtype}")
    g = torch.Generator(device="cuda").manual_seed(C)
    xt = torch.randint(0, 256, (N, H, W, C), dtype=torch.uint8, device="cuda", generator=g)
    mean, std = (0.485, 0.456, 0.406, 0.5)[:C], (0.229, 0.224, 0.225, 0.25)[:C]
    args = (mean, std, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 99)
    whole = torch.empty((N, H, W, oc), dtype=torch.float16, device="cuda")
    parts = torch.empty_like(whole)
    row, img = W * C, H * W * C
    b.fn_fused_normalize_ex(xt, row, img, N, H, W, C, *args, 0, out_dtype, whole)
    for a_ in range(0, N, 128):
        b_ = min(N, a_ + 128)
        b.fn_fused_normalize_ex(xt[a_:b_], row, img, b_ - a_, H, W, C, *args, a_, out_dtype,
                                parts[a_:b_])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), parts.view(torch.int16))


def test_long_strided_launch_equals_its_short_slices(b):
    """The same for a strided source: centre 224x224 windows of 256x256x3
    images, 1,030 of them (465 MB moved), against slices of 128 images."""
    N, S, H, W, C = 1030, 256, 224, 224, 3
    say(f"long strided launch: N={N}")
    g = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randint(0, 256, (N, S, S, C), dtype=torch.uint8, device="cuda", generator=g)
    row, img = S * C, S * S * C
    first = (16 * S + 16) * C
    args = (synth.IMAGENET_MEAN, synth.IMAGENET_STD, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 21)
    whole = torch.empty((N, H, W, C), dtype=torch.float16, device="cuda")
    parts = torch.empty_like(whole)
    base = src.data_ptr() + first
    b.fn_fused_normalize_ex(base, row, img, N, H, W, C, *args, 0, 1, whole)
    for a_ in range(0, N, 128):
        b_ = min(N, a_ + 128)
        b.fn_fused_normalize_ex(base + a_ * img, row, img, b_ - a_, H, W, C, *args, a_, 1,
                                parts[a_:b_])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), parts.view(torch.int16))


@pytest.mark.parametrize("first", [0, 1, 255, 2**32 - 3, 2**40 + 17])
def test_params_ex_bit_exact(b, first):
    N, H, W = 300, 224, 224
    say(f"params_ex: first={first}")
    t = torch.empty((N, 8), dtype=torch.int32, device="cuda")
    b.fn_params_ex(123, first, N, H, W, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, t)
    torch.cuda.synchronize()
    got = b.params_to_numpy(t)
    ref = oracle.params(123, first, N, H, W, 0.5, 0.5, (0.02, 0.33), (0.3, 3.3))
    assert got.tobytes() == ref.tobytes()


def test_centre_crop_workload_full_size(b):
    """The measured crop workload: 256 centre 224x224 windows of 256x256
    sources, fp16, ImageNet preset; exact RNE16 of the oracle on the
    windows, erased elements +0."""
    w = synth.WORKLOADS["imagenet_crop"]
    x = w.make_input()
    N, sh, sw, C = x.shape
    say(f"crop workload: {x.shape} -> {w.H}x{w.W} at ({w.y0}, {w.x0})")
    xt = torch.from_numpy(x).cuda()
    out = torch.empty(w.out_shape, dtype=torch.float16, device="cuda")
    seed = w.seeds[0]
    b.fn_fused_normalize_ex(xt.data_ptr() + (w.y0 * sw + w.x0) * C, sw * C, sh * sw * C, N, w.H,
                            w.W, C, w.mean, w.std, w.flip_p, w.erase_p, *w.scale, *w.ratio, seed,
                            0, w.out_dtype, out)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_normalize(w.window(x), w.mean, w.std, w.flip_p, w.erase_p, w.scale,
                                    w.ratio, seed=seed, threads=THREADS)
    check_values(out.cpu().numpy(), ref, "imagenet_crop")
