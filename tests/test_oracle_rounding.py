"""Pins of the rounding sequence of the oracle's erase attempt.

Page "(11) FusedNormalization": section 10 defines uniform(a, b) as
a + r (b - a) on floats, and section 12's generate_erase_rect() computes the
area fraction and the log aspect ratio that way, the aspect ratio with exp,
then each side as round(sqrt(area * ratio)) and round(sqrt(area / ratio)),
all in float.  The reading taken: every one of those float operations is
rounded to fp32 on its own (no fused multiply-add, no wider intermediate),
exp, sqrt and division are correctly rounded, and round() takes halves
away from zero.

The expected sides here are computed one operation at a time in exact
rational arithmetic (each step rounded to fp32 with ties to even; exp, ln
and sqrt from 60-digit decimals), independently of the oracle.  The cases
were picked so that a plausible other evaluation gives a different side:
  - fma_scale: fraction = fma(r, span, min), one rounding instead of two;
  - fma_log:   the log aspect ratio by the same fused form;
  - sqrt_double: sqrt of area*ratio (exact in double) and of area/ratio
    (rounded to double) taken in double and then rounded to fp32.
Each case asserts both that the oracle equals the one-rounding-per-operation
value and that the alternative evaluation differs from it, so an oracle
built either other way fails here.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from exact import exp_f32, ln_f32, nearest_f32, nearest_f64, round_half_away, sqrt_exact

IMAGENET_RANGES = ((0.02, 0.33), (0.3, 3.3))


def _r32(q: Fraction) -> Fraction:
    return Fraction(float(nearest_f32(q)))


def _arg(x: float) -> Fraction:
    """A float argument as it crosses the C ABI: its fp32 value."""
    return Fraction(float(np.float32(x)))


def attempt(ws: int, wr: int, H: int, W: int, scale=IMAGENET_RANGES[0], ratio=IMAGENET_RANGES[1],
            variant: str = "per_op"):
    """(eh, ew, fits) of one erase attempt from its area word ws and
    log-ratio word wr, in exact arithmetic with the stated roundings."""
    smin, smax = _arg(scale[0]), _arg(scale[1])
    lmin = Fraction(float(ln_f32(float(np.float32(ratio[0])))))
    lmax = Fraction(float(ln_f32(float(np.float32(ratio[1])))))
    u = Fraction(ws >> 8, 1 << 24)
    v = Fraction(wr >> 8, 1 << 24)
    img_area = _r32(Fraction(H) * Fraction(W))
    span = _r32(smax - smin)
    t = _r32(smin + u * span) if variant == "fma_scale" else _r32(smin + _r32(u * span))
    area = _r32(t * img_area)
    lspan = _r32(lmax - lmin)
    L = _r32(lmin + v * lspan) if variant == "fma_log" else _r32(lmin + _r32(v * lspan))
    ar = Fraction(float(exp_f32(float(L))))
    if variant == "sqrt_double":
        prod = area * ar                       # exact in double (two 24-bit significands)
        quot = Fraction(nearest_f64(area / ar))
        sh = _r32(Fraction(nearest_f64(sqrt_exact(prod))))
        sw = _r32(Fraction(nearest_f64(sqrt_exact(quot))))
    else:
        sh = _r32(sqrt_exact(_r32(area * ar)))
        sw = _r32(sqrt_exact(_r32(area / ar)))
    eh, ew = round_half_away(sh), round_half_away(sw)
    return eh, ew, (0 < eh < H and 0 < ew < W)


# (H, W, area word, log-ratio word, the alternative evaluation it separates)
CASES = [
    (224, 224, 2048291695, 2410041588, "fma_scale"),
    (224, 224, 3580136938, 281136026, "fma_scale"),
    (224, 224, 3614232171, 369454123, "fma_log"),
    (224, 224, 1918416915, 4194391372, "fma_log"),
    (224, 224, 2631243037, 3758375077, "sqrt_double"),
    (224, 224, 1342949223, 166376311, "sqrt_double"),
    (4096, 4096, 1437896968, 2547951252, "fma_scale"),
    (4096, 4096, 1067933765, 2587758268, "fma_log"),
    (4096, 4096, 843915409, 3865692934, "sqrt_double"),
    (4096, 4096, 206357128, 4014452702, "sqrt_double"),
    (300, 400, 3728649143, 85970669, "fma_scale"),
    (300, 400, 2653902478, 3719722258, "fma_log"),
    (300, 400, 2994763952, 4098675943, "sqrt_double"),
    (300, 400, 2790711167, 560544420, "sqrt_double"),
]


@pytest.mark.parametrize("H,W,ws,wr,other", CASES)
def test_attempt_rounds_each_operation_once(orc, H, W, ws, wr, other):
    want = attempt(ws, wr, H, W)
    alt = attempt(ws, wr, H, W, variant=other)
    assert alt != want, f"case does not separate {other}: {want}"
    assert orc.erase_dims(ws, wr, H, W) == want, (want, alt)


def test_exact_evaluator_agrees_with_closed_forms():
    """The evaluator itself, on cases with exact closed forms: ratio range
    [1, 1] gives ar = 1 and t = scale exactly, so the sides are
    round(sqrt(t H W))."""
    for t, H, W, side in [(0.0625, 10, 10, 3), (0.1225, 10, 10, 4), (0.25, 64, 64, 32),
                          (0.5, 2, 2, 1)]:
        eh, ew, fits = attempt(0, 0, H, W, scale=(t, t), ratio=(1.0, 1.0))
        assert (eh, ew) == (side, side)


@pytest.mark.parametrize("n,sides,other,alt_sides", [
    (618055, (41, 106), "fma_scale", (42, 106)),
    (668565, (176, 63), "fma_log", (176, 64)),
])
def test_whole_sample_needs_per_operation_rounding(orc, torch_philox, n, sides, other, alt_sides):
    """Seed 7, 224x224, flip 0.5, erase 1.0: the stream's words (from
    PyTorch's own Philox, not the oracle's) drive the draw of page section
    12; the accepted rectangle's sides with one rounding per operation
    differ from those of the fused evaluation."""
    seed, H, W = 7, 224, 224
    words = [int(w) for w in torch_philox(seed, n, 0, 24)]
    k = 2  # flip word, gate word (erase 1.0: the gate always opens)
    a = 0
    while True:
        eh, ew, fits = attempt(words[k], words[k + 1], H, W)
        if fits:
            break
        k += 2
        a += 1
    alt = attempt(words[k], words[k + 1], H, W, variant=other)
    i = (words[k + 2] * (H - eh + 1)) >> 32
    j = (words[k + 3] * (W - ew + 1)) >> 32
    flip = int((words[0] >> 8) < (1 << 23))  # u < 0.5
    P = orc.params(seed, n, 1, H, W, 0.5, 1.0)[0]
    assert (int(P["flip"]), int(P["erase"]), int(P["attempt"]), int(P["i"]), int(P["j"]),
            int(P["eh"]), int(P["ew"]), int(P["words_used"])) == (flip, 1, a, i, j, eh, ew,
                                                                 2 + 2 * a + 4)
    assert (eh, ew) == sides and alt[:2] == alt_sides
