"""The padded fp16 layout (FN_OUT_FP16_PAD4, page "(11) FusedNormalization",
section 8: four channels per pixel for mixed-precision training) through the
C ABI.  Pinned by the same oracle as the compact layout: channels c < C
within one fp16 ulp of the oracle (equal to RNE16(oracle) at the preset
constants), channels C..3 exactly +0, and channels c < C bit-identical to the
compact fp16 output of the same call arguments."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from augmentation_amd import synth

from test_gpu_parity import THREADS, check_values, say, wl_dict  # noqa: F401  (b fixture below)

pytestmark = pytest.mark.gpu

PAD4 = 2


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    return binding


def check_pad4(got4: np.ndarray, ref: np.ndarray, C: int, what: str, rne_exact: bool):
    assert got4.dtype == np.float16 and got4.shape[-1] == 4, what
    check_values(np.ascontiguousarray(got4[..., :C]), ref, what, rne_exact=rne_exact)
    pad = got4[..., C:].view(np.uint16)
    assert np.all(pad == 0), (what, int(np.count_nonzero(pad)))


@pytest.mark.parametrize("name", ["mnist", "cifar", "imagenet_train", "imagenet_val"])
def test_pad4_workloads(b, name):
    w = synth.WORKLOADS[name]
    x = w.make_input()
    seed = w.seeds[0]
    say(f"pad4: {name} {x.shape} seed={seed}")
    xt = torch.from_numpy(x).cuda()
    kw = wl_dict(w)
    args = (kw["mean"], kw["std"], kw["flip_p"], kw["erase_p"], kw["scale"], kw["ratio"], seed)
    o4 = b.fused_normalize(xt, *args[:2], flip_p=args[2], erase_p=args[3], scale=args[4],
                           ratio=args[5], seed=seed, out_dtype=PAD4)
    o16 = b.fused_normalize(xt, *args[:2], flip_p=args[2], erase_p=args[3], scale=args[4],
                            ratio=args[5], seed=seed, out_dtype=1)
    torch.cuda.synchronize()
    assert tuple(o4.shape) == (w.N, w.H, w.W, 4)
    ref, _ = oracle.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                    seed=seed, threads=THREADS)
    got4 = o4.cpu().numpy()
    check_pad4(got4, ref, w.C, name, rne_exact=True)
    assert np.array_equal(got4[..., :w.C].view(np.uint16), o16.cpu().numpy().view(np.uint16))


PAD4_SHAPES = [(3, 5, 7, 1), (2, 9, 5, 2), (4, 6, 5, 3), (2, 3, 3, 4), (1, 1, 1, 3),
               (1, 1, 17, 3), (5, 17, 1, 3), (3, 2, 2, 1), (2, 31, 33, 3), (7, 13, 12, 4),
               (2, 4, 4096, 1), (1, 600, 6, 3), (9, 28, 28, 1), (64, 32, 32, 3),
               (2, 3, 1024, 3), (2, 5, 700, 2), (40, 8, 8, 2), (3, 64, 48, 3),
               (1, 3, 9000, 3)]  # a 27 KB row: one-row tiles


@pytest.mark.parametrize("shape", PAD4_SHAPES)
@pytest.mark.parametrize("out_aligned", [True, False])
def test_pad4_edge_shapes_with_guards(b, shape, out_aligned):
    """Odd and even widths (even widths at a 16-byte aligned output take the
    tiles kernel, the rest the flat one), rows wider than one pass of the
    lanes, the input at a
    byte offset in 1..7, the output 16-byte aligned or only 2-byte aligned,
    and guard bands around the output."""
    N, H, W, C = shape
    rng = np.random.default_rng(7 * sum(shape))
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    mean = tuple(float(v) for v in rng.uniform(0.3, 0.6, C))
    std = tuple(float(v) for v in rng.uniform(0.2, 0.3, C))
    elems = N * H * W * C
    out_elems = N * H * W * 4
    in_off = 1 + (sum(shape) % 7)
    out_off = 4096 if out_aligned else 4096 + 2
    guard = 4096
    seed = 2000 + N + out_off
    say(f"pad4 edge: shape={shape} in_off={in_off} out_off={out_off}")
    in_buf = torch.zeros(elems + in_off + 64, dtype=torch.uint8, device="cuda")
    in_buf[in_off:in_off + elems] = torch.from_numpy(x.reshape(-1)).cuda()
    out_buf = torch.full((out_off + out_elems * 2 + guard,), 0xA5, dtype=torch.uint8,
                         device="cuda")
    b.fn_fused_normalize(in_buf.data_ptr() + in_off, N, H, W, C, mean, std, 0.5, 1.0, 0.02, 0.33,
                         0.3, 3.3, seed, PAD4, out_buf.data_ptr() + out_off)
    torch.cuda.synchronize()
    host = out_buf.cpu().numpy()
    assert np.all(host[:out_off] == 0xA5) and np.all(host[out_off + out_elems * 2:] == 0xA5)
    got = host[out_off:out_off + out_elems * 2].view(np.float16).reshape(N, H, W, 4)
    ref, _ = oracle.fused_normalize(x, mean, std, 0.5, 1.0, seed=seed)
    check_pad4(got, ref, C, str(shape), rne_exact=False)


def test_pad4_short_output_buffer_rejected(b):
    """The padded output needs N*H*W*4 elements: an allocation of exactly the
    compact size (straight from the HIP runtime, so no allocator slack) is
    rejected before any launch; one of the padded size is accepted."""
    import ctypes
    import os
    N, H, W, C = 2, 8, 8, 3
    x = torch.zeros((N, H, W, C), dtype=torch.uint8, device="cuda")
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    args = ((0.5,) * 3, (0.25,) * 3, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 1, PAD4)
    short, full = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(short), ctypes.c_size_t(N * H * W * C * 2)) == 0
    assert hip.hipMalloc(ctypes.byref(full), ctypes.c_size_t(N * H * W * 4 * 2)) == 0
    try:
        with pytest.raises(b.FnError) as e:
            b.fn_fused_normalize(x, N, H, W, C, *args, short.value)
        assert e.value.code == b.FN_EINVAL
        b.fn_fused_normalize(x, N, H, W, C, *args, full.value)
        torch.cuda.synchronize()
    finally:
        hip.hipFree(short)
        hip.hipFree(full)
