"""GPU parity of the decode path (append + absorbed split-S decode) against the
fp64 oracle, through the C ABI.  Tolerance: max relative error per output row
1e-2 for bf16 storage with fp32 accumulation, 1e-4 for the fp32 build."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from oracle import mla as O
from tests.helpers import DecodeCase, host, oracle_shape, row_rel_err, tol

pytestmark = pytest.mark.gpu


def _run_host(case, stages=True):
    """One decode of the case; (y, q_cat, o_lat) as host arrays (q_cat and
    o_lat None without stages)."""
    out = case.run(stages=stages)
    y, q_cat, o_lat = out if stages else (out, None, None)
    return host(y), (host(q_cat) if stages else None), (host(o_lat) if stages else None)


def _compare(case, out, bs, absorbed_only=()):
    """Compare y (and the staged q_cat / o_lat, when present) of every
    sequence in bs with the oracle; sequences in absorbed_only take y from
    the oracle's absorbed form."""
    y, q_cat, o_lat = out
    t = tol(case.dtype)
    for b in bs:
        y_ref, a = case.oracle(b, absorbed_only=b in absorbed_only)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < t, f"seq {b} (len {case.lens[b]}): y rel err {err:.3e}"
        if q_cat is not None:
            eq = row_rel_err(q_cat[b].reshape(1, -1), a["q_cat"][0].reshape(1, -1))[0]
            eo = row_rel_err(o_lat[b].reshape(1, -1), a["o_lat"][0].reshape(1, -1))[0]
            assert eq < t, f"seq {b}: q_cat rel err {eq:.3e}"
            assert eo < t, f"seq {b}: o_lat rel err {eo:.3e}"


def _check(case, bs, stages=True, absorbed_only=()):
    """Decode the case once and compare the sequences in bs with the oracle."""
    out = _run_host(case, stages)
    _compare(case, out, bs, absorbed_only)
    return out[0]


def full_size_case(workload, kv="dtype"):
    """A full-size ragged batch of a named workload, filled through the
    library's append and decoded once (staged) in the launch configuration
    the benchmark times: (case, host outputs)."""
    w = synth.WORKLOADS[workload]
    case = DecodeCase(w.dims, "bf16", w.weight_std, synth.lengths(w), random_gains=False, kv=kv,
                      absorb=w.absorb)
    out = _run_host(case, stages=True)
    assert all(np.all(np.isfinite(a)) for a in out)
    return case, out


def chunk(B, i, n=4):
    """Sequences of chunk i of n (every sequence is in exactly one chunk)."""
    return range(i * B // n, (i + 1) * B // n)


def test_tiny_f32_decode():
    """8 cached tokens at positions 0..7, decode at position 8; fp32 build."""
    w = synth.WORKLOADS["tiny_f32_decode"]
    case = DecodeCase(w.dims, "f32", w.weight_std, synth.lengths(w))
    _check(case, [0])


def test_tiny_f32_ragged():
    case = DecodeCase(synth.TINY, "f32", 0.05, [0, 1, 7, 16, 33, 100])
    _check(case, range(6))


def test_v2lite_ragged_small():
    """V2-Lite shapes (MFMA path): a single row, sub-tile boundaries (16),
    several waves' worth and a ragged tail."""
    lens = [0, 1, 14, 15, 16, 17, 63, 64, 65, 130, 700, 1500]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens)
    _check(case, range(len(lens)))


def test_v2lite_generic_path_bf16():
    """bf16 shapes outside the MFMA tiling (8 heads, latent 64) take the
    VALU kernels; same oracle, same tolerance."""
    dims = synth.LayerDims(hidden=256, n_heads=8, qk_nope=32, qk_rope=16, v_head=32,
                           kv_lora=64)
    case = DecodeCase(dims, "bf16", 0.05, [0, 5, 40, 300])
    _check(case, range(4))


def test_v2lite_decode_b1_s4096():
    """One sequence, 4096 cached rows + the decode token."""
    w = synth.WORKLOADS["v2lite_decode_b1_s4096"]
    case = DecodeCase(w.dims, "bf16", w.weight_std, synth.lengths(w), random_gains=False)
    _check(case, [0])


def test_v2lite_long_and_short_mixed():
    """One long sequence split over many workgroups (~46 partials, merged by
    eight waves in the fused combine) next to short ones, one of them
    finished by the core itself."""
    lens = [3000, 5, 40, 1, 700]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens)
    _check(case, range(len(lens)))


@pytest.mark.parametrize("n_short", [0, 127])
def test_combine_first_pass(n_short):
    """A sequence of 20,000 rows split over ~200 parts: more partials than the
    fused combine merges directly (128 with eight waves on the one sequence of
    a block, 16 with one wave per sequence at 128 sequences), so the chunked
    first pass runs before it.  The long sequence against the oracle's
    absorbed form (pinned equal to the non-absorbed one), a few short ones
    against the non-absorbed step."""
    lens = [20000] + [50 + 7 * i for i in range(n_short)]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, keep=[0, 1, n_short] if n_short else [0])
    _check(case, [0, 1, n_short] if n_short else [0], absorbed_only={0})


@pytest.fixture(scope="module")
def v2lite_b64():
    return full_size_case("v2lite_decode_b64")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_v2lite_decode_b64_full_size(v2lite_b64, part):
    """The full B=64 ragged batch (lengths ~ U{512..8192}), decoded once in
    the launch configuration the benchmark times: y, q_cat and o_lat of EVERY
    sequence against the oracle (y from the non-absorbed fp64 step), a
    quarter of the batch per test."""
    case, out = v2lite_b64
    _compare(case, out, chunk(case.B, part))


def test_v3_ragged_small():
    """V3 shapes (128 heads = 8 head groups, q LoRA 1536)."""
    case = DecodeCase(synth.V3, "bf16", 0.02, [0, 17, 250, 900])
    _check(case, range(4))


@pytest.fixture(scope="module")
def v3_b32():
    return full_size_case("v3_decode_b32")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_v3_decode_b32_full_size(v3_b32, part):
    """The full V3 B=32 ragged batch (cached lengths ~ U{2048..16384}),
    decoded once in the launch configuration of the many-head core: y, q_cat
    and o_lat of EVERY sequence against the oracle, a quarter per test.  y of
    the shortest sequence of each quarter comes from the non-absorbed fp64
    step; the others from the absorbed fp64 form (pinned equal to it at V3
    shapes), since expanding K and V for 128 heads over all 295k rows would
    take ~10 TFLOP of fp64."""
    case, out = v3_b32
    bs = list(chunk(case.B, part))
    full = {min(bs, key=lambda b: case.lens[b])}
    _compare(case, out, bs, absorbed_only=set(bs) - full)


def test_v3_decode_b1_s32768_long_context():
    """The long-context stress case of the V3 configuration: one sequence with
    32,768 cached rows plus the new one.  Against the oracle's absorbed form
    (pinned equal to the non-absorbed definition at V3 shapes; expanding K and
    V for 32k rows x 128 heads in fp64 would take gigabytes): q_cat, o_lat and
    y at the bf16 tolerance."""
    w = synth.WORKLOADS["v3_decode_b1_s32768"]
    lens = synth.lengths(w)
    assert int(lens[0]) == 32768
    case = DecodeCase(w.dims, "bf16", w.weight_std, lens, random_gains=False)
    y, q_cat, o_lat = case.run(stages=True)
    shp = oracle_shape(w.dims)
    L = int(lens[0])
    x = case.hidden[0]
    rows = O.latent_rows(x[:L + 1], np.arange(L + 1), case.w["w_kva"], case.w["kv_norm_g"], shp)
    ref = O.absorbed_step(x[L:L + 1], np.array([L]), rows, case.w, shp)
    t = tol("bf16")
    assert row_rel_err(host(y), ref["y"])[0] < t
    assert row_rel_err(host(q_cat).reshape(1, -1), ref["q_cat"].reshape(1, -1))[0] < t
    assert row_rel_err(host(o_lat).reshape(1, -1), ref["o_lat"].reshape(1, -1))[0] < t


def test_ring_core_two_head_groups():
    """32 heads: two 16-head workgroups per part of the ring core, on one XCD."""
    import dataclasses
    dims = dataclasses.replace(synth.V2_LITE, n_heads=32)
    case = DecodeCase(dims, "bf16", 0.02, [0, 40, 700, 2000])
    _check(case, range(4))


def test_value_head_64():
    """v_head = 64: the MFMA core with the separate combine and value GEMM."""
    import dataclasses
    dims = dataclasses.replace(synth.V2_LITE, v_head=64)
    case = DecodeCase(dims, "bf16", 0.02, [5, 300, 1200])
    _check(case, range(3))


def test_decode_is_deterministic():
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [300, 2000, 5])
    y1 = case.run().clone()
    y2 = case.run()
    assert bool((y1.view(dtype=y1.dtype) == y2).all())
    import torch
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_partials_fresh_across_calls():
    """Split partials are handed between workgroups (possibly on different
    XCDs) through the workspace; a second call on the same workspace with other
    sequences in the same slots must see its own partials, not the first
    call's.  The first batch is then decoded again and must be bit-identical."""
    a = DecodeCase(synth.V2_LITE, "bf16", 0.02, [3000, 900, 5, 1600])
    ya = a.run().clone()
    b = DecodeCase(synth.V2_LITE, "bf16", 0.02, [1600, 5, 3000, 900], layer=a.layer,
                   weights=a.w)
    _check(b, range(b.B), stages=False)
    ya2 = a.run()
    import torch
    assert torch.equal(ya.view(torch.int16), ya2.view(torch.int16))


def _step_case(dims, lens, std=0.02):
    """Cache holds only the cached rows; decode_step appends the new token
    itself and must match the oracle (and the append + decode path)."""
    import torch
    from tests.helpers import dev
    case = DecodeCase(dims, "bf16", std, lens)
    # wipe each sequence's new-token row, then let decode_step write it
    last = case.seq_off + case.seq_len - 1
    ref_rows = case.cache[torch.as_tensor(last, device="cuda")].clone()
    case.cache[torch.as_tensor(last, device="cuda")] = 0
    y = case.layer.decode_step(dev(case.x_new, torch.bfloat16), case.seq_off, case.seq_len,
                               case.cache)
    rows = case.cache[torch.as_tensor(last, device="cuda")]
    # same arithmetic up to the split-K summation order of the fused projection
    assert row_rel_err(host(rows), host(ref_rows)).max() < tol("bf16")
    y = host(y)
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol("bf16"), f"seq {b}: y rel err {err:.3e}"


def test_decode_step_v2lite():
    _step_case(synth.V2_LITE, [0, 1, 16, 63, 300, 1500])


def test_decode_step_v3():
    _step_case(synth.V3, [0, 40, 700])


def test_decode_step_batch_80():
    """80 tokens: the stream GEMMs with 64-row blocks (ragged last block)."""
    _step_case(synth.V2_LITE, [3 * b + (b % 7) * 11 for b in range(80)])


def test_decode_step_batch_136():
    """More than 128 tokens: the projections leave the stream GEMMs for the
    split-K tile GEMM path."""
    _step_case(synth.V2_LITE, [2 * b + (b % 5) * 13 for b in range(136)])


# A 256-head layer with a 1024-wide query LoRA and hidden 2048: its query
# up-projection (N = 256 * 192 = 49152, K = 1024, 96 MiB of weights) runs the
# resident-activation product in one K slice, with the epilogue applied in
# place; its output projection (N = 2048, K = 32768, 128 MiB) in 32 slices and
# the slice reduction (both past the 80 MiB from which the split-K products
# take over from the column tiles); its decode core runs two 128-head
# workgroups per part.
RES_DIMS = synth.LayerDims(hidden=2048, n_heads=256, qk_nope=128, qk_rope=64, v_head=128,
                           kv_lora=512, q_lora=1024)


def test_resident_products_one_and_many_slices():
    case = DecodeCase(RES_DIMS, "bf16", 0.02, [0, 33, 400])
    _check(case, range(3))


def test_decode_step_resident_one_slice():
    _step_case(RES_DIMS, [5, 90, 300])


def test_core_timing_ring():
    """The library's core-launch timing: a ring of 3 slots after 5 decodes
    holds the last 3 durations, each positive and below a second."""
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [300, 40])
    case.layer.core_timing(3)
    for _ in range(5):
        case.run(stages=False)
    ms = case.layer.core_timing_read(10)
    case.layer.core_timing(0)
    assert len(ms) == 3
    assert np.all(ms > 0) and np.all(ms < 1000)
    assert len(case.layer.core_timing_read(10)) == 0
