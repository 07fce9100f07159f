"""GPU parity of materialised absorption (mla_config.absorb =
MLA_ABSORB_MATERIALIZED: W^KQ_h = W_UK_h^T W_q,nope_h and W^OV_h = W_o,h W_UV_h
formed once, "Multi-Head Latent Attention" post, section 3.5), through the C
ABI, against the fp64 non-absorbed oracle at the bf16 tolerance: the staged
q_cat and o_lat and the output y of every sequence."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from tests.helpers import DecodeCase, dev, host, row_rel_err, tol
from tests.test_gpu_decode import _check, _compare, chunk, full_size_case

pytestmark = pytest.mark.gpu


def test_materialized_decode_ragged_small():
    lens = [0, 1, 33, 64, 700, 1500]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, absorb="materialized")
    _check(case, range(len(lens)))


def test_materialized_query_lora_layer():
    """128 heads with a query LoRA: W^KQ_h = W_UK_h^T W_qb,nope_h (d_c x q_lora)."""
    lens = [0, 40, 700]
    case = DecodeCase(synth.V3, "bf16", 0.02, lens, absorb="materialized")
    _check(case, range(len(lens)))


@pytest.mark.parametrize("dims", [synth.V2_LITE, synth.V3], ids=["v2lite", "v3"])
def test_materialized_decode_step(dims):
    """decode_step appends the new rows from the same in-projection that forms
    q_abs, then decodes them."""
    import torch
    case = DecodeCase(dims, "bf16", 0.02, [3, 40, 1500], absorb="materialized")
    y = host(case.layer.decode_step(dev(case.x_new, torch.bfloat16), case.seq_off, case.seq_len,
                                    case.cache))
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol("bf16"), f"seq {b}: y rel err {err:.3e}"


def test_materialized_agrees_with_factored():
    """Both forms of the same layer on the same cache give the same outputs to
    the bf16 tolerance."""
    import torch
    from tests.helpers import make_layer
    lens = [5, 300, 2000, 64]
    a = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, absorb="materialized", keep=[])
    f = make_layer(synth.V2_LITE, "bf16", a.w)
    x = dev(a.x_new, torch.bfloat16)
    ya = host(a.layer.decode(x, a.seq_len - 1, a.seq_off, a.seq_len, a.cache))
    yf = host(f.decode(x, a.seq_len - 1, a.seq_off, a.seq_len, a.cache))
    assert row_rel_err(ya, yf).max() < tol("bf16")


def test_materialized_large_batch_uses_factored_weights():
    """Beyond the fused path's 128 query rows the handle decodes with its
    factored weights; results still match the oracle."""
    lens = [(7 * b) % 50 for b in range(130)]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, absorb="materialized",
                      keep=[0, 1, 64, 129])
    _check(case, [0, 1, 64, 129])


@pytest.fixture(scope="module")
def mat_b64():
    return full_size_case("v2lite_decode_b64_materialized")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_materialized_decode_b64_full_size(mat_b64, part):
    """The benchmark's B=64 ragged batch with materialised weights: every
    sequence against the oracle, a quarter of the batch per test."""
    case, out = mat_b64
    _compare(case, out, chunk(case.B, part))
