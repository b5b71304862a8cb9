"""bench.py's command line on a machine without a GPU: it measures one GPU
only, and rejects malformed shape arguments before touching a device."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from conftest import ROOT


def run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=e, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run(*args, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args,message", [
    (["--shape", "1,2,3"], "--shape takes N,H,W,C"),
    (["--shape", "1,2,x,3"], "--shape takes N,H,W,C"),
    (["--shape", "0,224,224,3"], "--shape takes N,H,W,C"),
    (["--shape", "1,8,8,3", "--out", "fp32", "--out-offset", "2"], "--out-offset"),
    (["--shape", "1,8,8,3", "--out-offset", "16"], "--out-offset"),
])
def test_malformed_shape_arguments_are_refused(args, message):
    r = run(*args)
    assert r.returncode == 2
    assert message in r.stderr


def test_timeline_summary_of_synthetic_stamps():
    """bench.py --timeline's analysis on stamps with a known answer: four
    tiles that start together, stage for 2 us, issue their stores 1 us later
    and see them acknowledged 1 us after that."""
    import numpy as np
    import bench
    d = np.array([[1000, 1200, 1300, 1400]] * 4)  # ticks of 0.01 us
    r = bench.timeline_summary([d, d + 7], in_tile=1e6, out_tile=2e6)
    assert r["span"] == (4.0, 4.0, 4.0)
    assert r["stage"] == (2.0, 2.0, 2.0) and r["compute"] == (1.0, 1.0, 1.0)
    assert r["drain"] == (1.0, 1.0, 1.0) and r["life"] == (4.0, 4.0, 4.0)
    assert list(r["occupancy"]) == [4] * 8 + [0]
    assert r["first_generation"] == 4 and list(r["first_generation_retire"]) == [4.0] * 3
    assert r["last_start"] == 0.0 and r["tail_below_half"] == 0.5
    # 4 x 3 MB over 4 us; the middle half reads 1-2 us and writes 2-3 us
    assert abs(r["tbs_span"] - 3.0) < 1e-9 and abs(r["tbs_middle"] - 3.0) < 1e-9
