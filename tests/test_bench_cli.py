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
