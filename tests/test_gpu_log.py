"""MLA_LOG=1: the library prints one line per call on stderr with the call's
shape, the work plan and the kernels chosen (read once per process, so the
check runs in a child process with the variable set)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import torch
from mla_latent_kv_decode_amd import synth
from tests.helpers import DecodeCase
case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [5, 70])
case.run()
torch.cuda.synchronize()
print("child done", flush=True)
"""


@pytest.mark.timeout(240)
def test_log_lines():
    env = dict(os.environ, MLA_LOG="1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=200)
    assert r.returncode == 0 and "child done" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[mla] ")]
    assert any(l.startswith("[mla] create:") and "decode_core_ring_k" in l for l in lines), lines
    dec = [l for l in lines if l.startswith("[mla] decode:")]
    assert dec and "B=2" in dec[-1] and "rows=77" in dec[-1] and "parts" in dec[-1], lines


@pytest.mark.timeout(120)
def test_log_is_off_by_default():
    env = {k: v for k, v in os.environ.items() if k != "MLA_LOG"}
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=100)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "[mla] " not in r.stderr
