"""GPU parity of the FP8 latent cache (OCP E4M3 codes with one fp32 scale per
row, rope in bf16: 656-byte rows), through the C ABI.

* The store of given bf16 rows is bit-exact against the oracle's fp32
  decision path on the same values (codes, rope bits, scale bits, zero pad).
* The append and the decode step are compared with the fp64 oracle whose
  cache hands back its own quantised rows (oracle.fp8.fp8_rows); outputs to
  the bf16 tolerance, max relative error 1e-2 per row."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from oracle import fp8 as F8
from oracle import mla as O
from tests.helpers import DecodeCase, dev, host, make_layer, oracle_shape, row_rel_err, tol
from tests.test_gpu_decode import _check, _compare, chunk, full_size_case

pytestmark = pytest.mark.gpu

RB = 656  # bytes per FP8 row for kv_lora 512, qk_rope 64


def _split(rows_u8):
    """(codes (T, 512) uint8, rope (T, 64) float64, scale (T,) float64, pad)"""
    r = np.ascontiguousarray(rows_u8, dtype=np.uint8)
    rope_bits = r[:, 512:640].copy().view(np.uint16).astype(np.uint32) << 16
    rope = rope_bits.view(np.float32).astype(np.float64)
    scale = r[:, 640:644].copy().view(np.float32)[:, 0].astype(np.float64)
    return r[:, :512], rope, scale, r[:, 644:]


def test_fp8_store_is_bit_exact():
    import torch
    from mla_latent_kv_decode_amd.lib import MLALayer
    layer = MLALayer(synth.V2_LITE, "bf16", kv="fp8")
    assert layer.row_bytes() == RB
    rng = np.random.default_rng(11)
    T = 37
    mags = np.exp(rng.uniform(np.log(1e-4), np.log(300.0), T)).astype(np.float32)
    rows = rng.standard_normal((T, 576)).astype(np.float32) * mags[:, None]
    rows[3, :512] = 0.0                               # an all-zero latent
    rows[5, :512] = rng.integers(-8, 9, 512) * 0.25   # exact grid values
    rows = synth.bf16_round(rows)
    slot = rng.permutation(100)[:T]
    cache = layer.new_cache(100)
    layer.cache_store(dev(rows, torch.bfloat16), slot, cache)
    got = cache.cpu().numpy()
    s, q = F8.quantize_latent(rows[:, :512], f32=True)
    want_rope = (rows[:, 512:].view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
    for i, sl in enumerate(slot):
        assert np.array_equal(got[sl, :512], q[i]), i
        assert np.array_equal(got[sl, 512:640], want_rope[i].reshape(-1)), i
        assert got[sl, 640:644].tobytes() == np.float32(s[i]).tobytes(), i
        assert not got[sl, 644:].any()
    other = np.setdiff1d(np.arange(100), slot)
    assert not got[other].any()


def test_fp8_append_matches_oracle():
    import torch
    d = synth.V2_LITE
    w = synth.make_weights(d, 0.02, "bf16", random_gains=True)
    layer = make_layer(d, "bf16", w, kv="fp8")
    T = 300
    x = synth.hidden_states(3, T, d.hidden, "bf16")
    slot = 7 + 2 * np.arange(T)
    cache = layer.new_cache(2 * T + 10)
    layer.append(dev(x, torch.bfloat16), np.arange(T), slot, cache)
    got = cache.cpu().numpy()
    codes, rope, scale, pad = _split(got[slot])
    shp = oracle_shape(d)
    ref = O.latent_rows(x, np.arange(T), w["w_kva"], w["kv_norm_g"], shp)
    s_ref, q_ref = F8.quantize_latent(ref[:, :512])
    assert np.max(np.abs(scale / s_ref - 1)) < 1e-4
    # codes: the same E4M3 value, or the neighbouring one where the fp32 and
    # fp64 latents straddle a rounding midpoint
    back = scale[:, None] * F8.e4m3_decode(codes)
    back_ref = F8.dequantize_latent(s_ref, q_ref)
    same = codes == q_ref
    assert same.mean() > 0.99
    step = np.abs(back_ref) * 2.0 ** -3 + s_ref[:, None] * 2.0 ** -9
    assert np.all(np.abs(back - back_ref)[~same] <= step[~same] * 1.01)
    assert row_rel_err(rope, ref[:, 512:]).max() < tol("bf16")
    assert not pad.any()
    untouched = np.setdiff1d(np.arange(cache.shape[0]), slot)
    assert not got[untouched].any()


def test_fp8_decode_ragged_small():
    lens = [0, 1, 14, 31, 32, 33, 63, 64, 65, 130, 700, 1500]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, kv="fp8")
    _check(case, range(len(lens)))


def test_fp8_ring_core_two_head_groups():
    import dataclasses
    dims = dataclasses.replace(synth.V2_LITE, n_heads=32)
    case = DecodeCase(dims, "bf16", 0.02, [0, 40, 700, 2000], kv="fp8")
    _check(case, range(4))


@pytest.fixture(scope="module")
def fp8_b64():
    return full_size_case("v2lite_decode_b64", kv="fp8")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_fp8_decode_b64_full_size(fp8_b64, part):
    """The benchmark's B=64 ragged batch on an FP8 cache, decoded once: y,
    q_cat and o_lat of EVERY sequence against the oracle reading its own
    quantised rows, a quarter of the batch per test."""
    case, out = fp8_b64
    _compare(case, out, chunk(case.B, part))


@pytest.mark.parametrize("lens", [[0, 1, 16, 63, 300, 1500],
                                  [3 * b + (b % 7) * 11 for b in range(80)]])
def test_fp8_decode_step(lens):
    """decode_step appends the new tokens' FP8 rows itself (the fused
    projection path for B <= 64, the split-K path beyond) and decodes them."""
    import torch
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, kv="fp8")
    last = torch.as_tensor(case.seq_off + case.seq_len - 1, device="cuda")
    ref_rows = case.cache[last].clone()
    case.cache[last] = 0
    y = case.layer.decode_step(dev(case.x_new, torch.bfloat16), case.seq_off, case.seq_len,
                               case.cache)
    codes, rope, scale, _ = _split(case.cache[last].cpu().numpy())
    rcodes, rrope, rscale, _ = _split(ref_rows.cpu().numpy())
    # the same rows as the append path, up to the projection's summation order
    assert np.max(np.abs(scale / rscale - 1)) < 1e-4
    assert (codes == rcodes).mean() > 0.99
    assert row_rel_err(rope, rrope).max() < tol("bf16")
    y = host(y)
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol("bf16"), f"seq {b}: y rel err {err:.3e}"


def test_fp8_v3_decode_ragged_small():
    """A 128-head layer (q-LoRA, V3 shapes) on an FP8 cache: the many-head
    core decodes each raw tile once for all 128 heads; an empty sequence, a
    single row, ragged tails and several tiles."""
    lens = [0, 1, 33, 64, 700, 2000]
    case = DecodeCase(synth.V3, "bf16", 0.02, lens, kv="fp8")
    _check(case, range(len(lens)))


def test_fp8_v3_decode_step():
    """The V3 step appends FP8 rows through the q-LoRA projection path."""
    import torch
    case = DecodeCase(synth.V3, "bf16", 0.02, [3, 40, 1500], kv="fp8")
    y = host(case.layer.decode_step(dev(case.x_new, torch.bfloat16), case.seq_off, case.seq_len,
                                    case.cache))
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol("bf16"), f"seq {b}: y rel err {err:.3e}"


@pytest.fixture(scope="module")
def fp8_v3_b32():
    return full_size_case("v3_decode_b32", kv="fp8")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_fp8_v3_decode_b32_full_size(fp8_v3_b32, part):
    """The V3 B=32 ragged batch on an FP8 cache: y, q_cat and o_lat of every
    sequence against the oracle, a quarter of the batch per test."""
    case, out = fp8_v3_b32
    _compare(case, out, chunk(case.B, part))
