"""Seeded synthetic inputs for FusedNormalization.

This module is shared by the tests (on both sides of a parity check), the
smoke check and the benchmark.  It holds none of the method's arithmetic:
it only makes uint8 images and names the argument sets of five workloads.
The parameter-draw seed is an argument of the operation itself; nothing
random that the operation draws is made here.

The workloads follow the shapes, value ranges and presets the pages train
on (page "(11) FusedNormalization", section 9 presets; page "(25)" MNIST
and ImageNet experiments).  No dataset is read: the images are i.i.d.
uniform bytes, or, for the ImageNet-train shape, smooth per-image gradients
plus noise so that a horizontal flip is visible.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Presets of page "(11) FusedNormalization", section 9 (get_params).
MNIST_MEAN, MNIST_STD = (0.1307,), (0.3081,)
CIFAR_MEAN, CIFAR_STD = (0.4914, 0.4822, 0.4465), (0.2470, 0.2435, 0.2616)
IMAGENET_MEAN, IMAGENET_STD = (0.485, 0.456, 0.406), (0.229, 0.224, 0.225)

# RandomErasing defaults of page "(11)", section 4 (Preprocessor).
ERASE_SCALE = (0.02, 0.33)
ERASE_RATIO = (0.3, 3.3)

# The pages seed their experiments with manual_seed(123).
PARAM_SEED = 123

OUT_FP32, OUT_FP16, OUT_FP16_PAD4 = 0, 1, 2


def uniform_images(rng: np.random.Generator, N: int, H: int, W: int, C: int) -> np.ndarray:
    """i.i.d. uniform bytes in [0, 255]."""
    return rng.integers(0, 256, size=(N, H, W, C), dtype=np.uint8)


def gradient_images(rng: np.random.Generator, N: int, H: int, W: int, C: int) -> np.ndarray:
    """Per image and channel: a + gy*h/(H-1) + gx*w/(W-1), rounded, plus
    integer noise in [-16, 16], clipped to [0, 255]."""
    a = rng.uniform(0.0, 255.0, size=(N, 1, 1, C))
    gy = rng.uniform(-128.0, 128.0, size=(N, 1, 1, C))
    gx = rng.uniform(-128.0, 128.0, size=(N, 1, 1, C))
    hh = (np.arange(H, dtype=np.float64) / max(H - 1, 1)).reshape(1, H, 1, 1)
    ww = (np.arange(W, dtype=np.float64) / max(W - 1, 1)).reshape(1, 1, W, 1)
    out = np.empty((N, H, W, C), np.uint8)
    for n in range(N):  # one image at a time keeps the float64 temporaries small
        v = np.rint(a[n:n + 1] + gy[n:n + 1] * hh + gx[n:n + 1] * ww)
        v += rng.integers(-16, 17, size=(1, H, W, C))
        out[n] = np.clip(v, 0, 255).astype(np.uint8)[0]
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    W: int
    C: int
    mean: tuple
    std: tuple
    flip_p: float
    erase_p: float
    out_dtype: int
    data_seed: int
    kind: str = "uniform"          # "uniform" | "gradient"
    scale: tuple = ERASE_SCALE
    ratio: tuple = ERASE_RATIO
    seeds: tuple = field(default=(PARAM_SEED,))  # one launch per seed, same input
    # source images larger than H x W: the operation reads the H x W window
    # at (y0, x0) of each src_h x src_w image (0: the source is H x W)
    src_h: int = 0
    src_w: int = 0
    y0: int = 0
    x0: int = 0

    @property
    def launches(self) -> int:
        return len(self.seeds)

    @property
    def elems(self) -> int:
        return self.N * self.H * self.W * self.C

    @property
    def out_bytes(self) -> int:
        return 4 if self.out_dtype == OUT_FP32 else 2

    @property
    def out_channels(self) -> int:
        return 4 if self.out_dtype == OUT_FP16_PAD4 else self.C

    @property
    def out_shape(self) -> tuple:
        return (self.N, self.H, self.W, self.out_channels)

    @property
    def nominal_bytes(self) -> int:
        """Bytes one launch moves by the metric's count: every input byte
        read once and every output element written once, erased or not."""
        return self.elems + self.N * self.H * self.W * self.out_channels * self.out_bytes

    @property
    def source_shape(self) -> tuple:
        return (self.N, self.src_h or self.H, self.src_w or self.W, self.C)

    def make_input(self) -> np.ndarray:
        """The whole source batch (N, src_h, src_w, C) uint8, from the
        workload's data seed."""
        rng = np.random.default_rng(self.data_seed)
        N, sh, sw, C = self.source_shape
        if self.kind == "gradient":
            return gradient_images(rng, N, sh, sw, C)
        return uniform_images(rng, N, sh, sw, C)

    def window(self, x: np.ndarray) -> np.ndarray:
        """The H x W windows the operation reads, as a compact array."""
        return np.ascontiguousarray(x[:, self.y0:self.y0 + self.H, self.x0:self.x0 + self.W])


WORKLOADS = {
    "mnist": Workload("mnist", 200, 28, 28, 1, MNIST_MEAN, MNIST_STD, 0.5, 0.0, OUT_FP32, 1001),
    "cifar": Workload("cifar", 256, 32, 32, 3, CIFAR_MEAN, CIFAR_STD, 0.5, 0.5, OUT_FP32, 1002),
    "imagenet_train": Workload("imagenet_train", 256, 224, 224, 3, IMAGENET_MEAN, IMAGENET_STD,
                               0.5, 0.5, OUT_FP16, 1003, kind="gradient"),
    "imagenet_val": Workload("imagenet_val", 256, 224, 224, 3, IMAGENET_MEAN, IMAGENET_STD,
                             0.0, 0.0, OUT_FP32, 1004),
    "stress": Workload("stress", 2048, 224, 224, 3, IMAGENET_MEAN, IMAGENET_STD, 0.5, 1.0,
                       OUT_FP16, 1005, seeds=tuple(range(PARAM_SEED, PARAM_SEED + 8))),
    # the training batch read as centre 224x224 windows of 256x256 sources
    # (the crop that precedes the fused step, page "(11)" section 4)
    "imagenet_crop": Workload("imagenet_crop", 256, 224, 224, 3, IMAGENET_MEAN, IMAGENET_STD,
                              0.5, 0.5, OUT_FP16, 1006, kind="gradient", src_h=256, src_w=256,
                              y0=16, x0=16),
    # the training batch in the page's 4-channel mixed-precision layout (section 8)
    "imagenet_train_pad4": Workload("imagenet_train_pad4", 256, 224, 224, 3, IMAGENET_MEAN,
                                    IMAGENET_STD, 0.5, 0.5, OUT_FP16_PAD4, 1003, kind="gradient"),
}

# The workload the headline metric is quoted on.
HEADLINE = "imagenet_train"
