"""The instrumented build libfn_timeline.so (FN_TIMELINE=1) used by
`bench.py --timeline`: its outputs equal the product library's bit for
bit, and every tile of a launch leaves four ordered clock stamps."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from augmentation_amd import synth

from test_gpu_parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from augmentation_amd import binding
    if not os.path.exists(binding.TIMELINE_LIB_PATH):
        pytest.skip("libfn_timeline.so is not built")
    return binding


@pytest.mark.parametrize("N,out_dtype", [(32, 1), (7, 0), (5, 2)])
def test_instrumented_build_stores_the_same_bits(b, N, out_dtype):
    w = synth.WORKLOADS["imagenet_train"]
    say(f"timeline build: N={N} out_dtype={out_dtype}")
    x = torch.from_numpy(w.make_input()[:N]).cuda()
    L = b.timeline_library()
    tiles = N * w.H
    stamps = torch.zeros(tiles * 4, dtype=torch.int64, device="cuda")
    assert L.fn_test_timeline(stamps.data_ptr(), tiles) == 0
    oc = 4 if out_dtype == 2 else w.C
    tdt = torch.float32 if out_dtype == 0 else torch.float16
    ref = torch.empty((N, w.H, w.W, oc), dtype=tdt, device="cuda")
    got = torch.empty_like(ref)
    args = (w.mean, w.std, 0.5, 0.5, 0.02, 0.33, 0.3, 3.3, 5, out_dtype)
    b.fn_fused_normalize(x, N, w.H, w.W, w.C, *args[:-2], args[-2], args[-1], ref)
    mean, std = b._host_floats(w.mean, w.C), b._host_floats(w.std, w.C)
    rc = L.fn_fused_normalize(x.data_ptr(), N, w.H, w.W, w.C, mean, std, 0.5, 0.5, 0.02, 0.33,
                              0.3, 3.3, 5, out_dtype, got.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0, L.fn_last_error()
    torch.cuda.synchronize()
    assert L.fn_test_timeline(None, 0) == 0
    view = torch.int32 if out_dtype == 0 else torch.int16
    assert torch.equal(ref.view(view), got.view(view))
    d = stamps.view(-1, 4).cpu().numpy()
    used = d[:, 0] != 0
    # whole rows per tile: at least ceil(N * H / rows per tile) tiles, and
    # recorded tiles form a prefix of the index range
    n_used = int(used.sum())
    assert n_used >= 1 and used[:n_used].all() and not used[n_used:].any()
    d = d[:n_used]
    assert np.all(d[:, 0] <= d[:, 1]) and np.all(d[:, 1] <= d[:, 2]) and np.all(d[:, 2] <= d[:, 3])
    span_us = (d[:, 3].max() - d[:, 0].min()) * 0.01
    assert 0 < span_us < 1e5
