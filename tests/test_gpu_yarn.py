"""GPU parity with YaRN-interpolated RoPE frequencies (mla_config.rope_scale >
1), through the C ABI: decode (the step's fused projection path included) and
chunked prefill at positions past the original context, against the fp64
oracle using the same frequencies (oracle.mla.rope_theta)."""

import dataclasses

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from tests.helpers import DecodeCase, dev, host, row_rel_err, tol
from tests.test_gpu_decode import _check
from tests.test_gpu_prefill import run_prefill_case

pytestmark = pytest.mark.gpu

# DeepSeek-V2-Lite's context extension: 4k original positions, factor 40, the
# attention factor's coefficient 0.707 (the library derives the softmax scale)
YARN = dict(rope_scale=40.0, rope_orig_max=4096, yarn_beta_fast=32.0, yarn_beta_slow=1.0,
            yarn_mscale=0.707)


def test_yarn_decode_past_original_context():
    dims = dataclasses.replace(synth.V2_LITE, **YARN)
    case = DecodeCase(dims, "bf16", 0.02, [0, 31, 700, 4095, 4200, 9000])
    _check(case, range(6))


def test_yarn_decode_step():
    import torch
    dims = dataclasses.replace(synth.V2_LITE, **YARN)
    case = DecodeCase(dims, "bf16", 0.02, [3, 5000, 8191])
    y = host(case.layer.decode_step(dev(case.x_new, torch.bfloat16), case.seq_off, case.seq_len,
                                    case.cache))
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        assert row_rel_err(y[b:b + 1], y_ref[None])[0] < tol("bf16"), b


def test_yarn_prefill():
    dims = dataclasses.replace(synth.V2_LITE, **YARN)
    run_prefill_case(dims, "bf16", 0.02, [0, 4090], [70, 40])


def test_yarn_changes_the_result():
    """The frequencies reach the kernels: the same inputs decoded with plain
    RoPE differ from the YaRN result at long positions."""
    import torch
    lens = [6000]
    a = DecodeCase(dataclasses.replace(synth.V2_LITE, **YARN), "bf16", 0.02, lens, keep=[])
    b = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, keep=[])
    ya, yb = host(a.run()), host(b.run())
    assert row_rel_err(ya, yb)[0] > 1e-2
