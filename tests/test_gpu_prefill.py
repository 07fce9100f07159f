"""GPU parity of causal chunked prefill against the fp64 oracle: every new token
attends to its own sequence's rows up to its position (cached prefix + the
new tokens before it)."""

import types

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from oracle import fp8 as F8
from oracle import mla as O
from tests.helpers import dev, fill_sequence, host, make_layer, oracle_shape, row_rel_err, tol

pytestmark = pytest.mark.gpu


def prefill_inputs(dims, dtype, std, prior, new, kv="dtype", gap=0):
    """A chunked-prefill batch: sequence b owns cache rows [seq_off[b],
    seq_off[b] + prior[b] + new[b]) (gap free rows between sequences), all of
    them appended through the library first; returns the layer, weights,
    cache, hidden states and offsets."""
    import torch
    w = synth.make_weights(dims, std, dtype, random_gains=True)
    layer = make_layer(dims, dtype, w, kv=kv)
    prior = np.asarray(prior, np.int64)
    new = np.asarray(new, np.int64)
    tot = prior + new
    seq_off = np.concatenate([[0], np.cumsum(tot + gap)[:-1]]).astype(np.int64)
    cu_new = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    cache = layer.new_cache(int((tot + gap).sum()))
    hidden = []
    for b in range(len(prior)):
        x, _ = fill_sequence(layer, dims, dtype, b, int(tot[b]), cache, int(seq_off[b]),
                             keep=True)
        hidden.append(x)
    x_new = np.concatenate([hidden[b][prior[b]:] for b in range(len(prior))])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return types.SimpleNamespace(dims=dims, dtype=dtype, kv=kv, w=w, layer=layer, prior=prior,
                                 new=new, tot=tot, seq_off=seq_off, cu_new=cu_new, cache=cache,
                                 hidden=hidden, x_new=x_new, x_dev=dev(x_new, tdt))


def check_prefill(c, y, query_subset=None):
    """Rows of y (host) against the fp64 oracle (reading FP8 rows back as the
    cache stores them); returns the worst per-row relative error."""
    shp = oracle_shape(c.dims)
    rows_prior = [O.latent_rows(c.hidden[b][:c.prior[b]], np.arange(c.prior[b]), c.w["w_kva"],
                                c.w["kv_norm_g"], shp) if c.prior[b] else np.zeros((0, shp.row))
                  for b in range(len(c.prior))]
    store = (lambda r: F8.fp8_rows(r, shp.kv_lora)) if c.kv == "fp8" else None
    ref = O.prefill_batch(c.x_new, c.cu_new, c.prior, rows_prior, c.w, shp,
                          query_subset=query_subset, kv_store=store)
    worst = 0.0
    for b, (idx, yr) in enumerate(ref):
        err = row_rel_err(y[c.cu_new[b] + idx], yr)
        worst = max(worst, float(err.max()))
        assert err.max() < tol(c.dtype), (b, int(idx[np.argmax(err)]), float(err.max()))
    return worst


def run_prefill_case(dims, dtype, std, prior, new, query_subset=None, kv="dtype", gap=0):
    c = prefill_inputs(dims, dtype, std, prior, new, kv=kv, gap=gap)
    y = host(c.layer.prefill(c.x_dev, c.cu_new, c.prior.astype(np.int32), c.seq_off, c.cache))
    return check_prefill(c, y, query_subset)


def test_tiny_f32_prefill():
    run_prefill_case(synth.TINY, "f32", 0.05, [0, 3, 8], [9, 6, 1])


def test_v2lite_prefill_small():
    run_prefill_case(synth.V2_LITE, "bf16", 0.02, [0, 37, 100], [40, 13, 1])


def test_v2lite_prefill_multi_tile():
    """Several 256-query tiles and 32-key tiles per sequence, ragged tails,
    a 1-token chunk and a long prior."""
    run_prefill_case(synth.V2_LITE, "bf16", 0.02, [0, 300, 33], [600, 70, 1])


def test_v3_prefill_small():
    run_prefill_case(synth.V3, "bf16", 0.02, [0, 21], [24, 9])


@pytest.mark.timeout(300)
def test_v3_prefill_ragged_large_tiles():
    """5,500 new tokens and 6,500 key rows (neither a multiple of the 256-row
    GEMM tile): every projection and the expansion run on the large-tile
    GEMM with a ragged last row tile; sampled queries of both sequences,
    including the last ones."""
    q0 = np.unique(np.concatenate([np.arange(0, 3000, 97), np.arange(2990, 3000)]))
    q1 = np.unique(np.concatenate([np.arange(0, 2500, 89), np.arange(2490, 2500)]))
    run_prefill_case(synth.V3, "bf16", 0.02, [0, 1000], [3000, 2500], query_subset=[q0, q1])


@pytest.mark.timeout(600)
def test_v3_prefill_4x4096_full_size():
    """The V3 chunked prefill at its full size (4 sequences x 4096 new tokens
    after 0 / 2048 / 0 / 2048 cached rows) in the launch configuration the
    timing uses (mla_prefill_step: the fused in-projection and append, then
    the prefill): the 16,384 appended rows against mla_append_latent's, and
    every 64th query, the tile and key-tile edges and the whole last 256-query
    tile of every sequence against the oracle."""
    w = synth.WORKLOADS["v3_prefill_4x4096"]
    prior, new = [0, 2048, 0, 2048], [4096] * 4
    q = np.unique(np.concatenate([np.arange(0, 4096, 64), [1, 31, 32, 255, 256, 2047],
                                  np.arange(4096 - 256, 4096)]))
    run_step_case(w.dims, "bf16", w.weight_std, prior, new, query_subset=[q] * 4)


def test_v2lite_fp8_prefill():
    """An FP8 cache: the key rows are decoded to bf16 before the expansion;
    against the oracle reading its own quantised rows.  Gaps between the
    sequences' rows exercise the gather's source offsets."""
    run_prefill_case(synth.V2_LITE, "bf16", 0.02, [0, 300, 33], [600, 70, 1], kv="fp8", gap=5)


def test_v3_fp8_prefill_small():
    run_prefill_case(synth.V3, "bf16", 0.02, [0, 21], [24, 9], kv="fp8")


def run_step_case(dims, dtype, std, prior, new, kv="dtype", gap=0, query_subset=None):
    """mla_prefill_step against the same batch appended through
    mla_append_latent: the step must write the new tokens' latent rows (the
    same rows up to the summation order of the fused in-projection, or the
    same FP8 codes but for rare rounding ties), leave every other cache row
    alone, and give the oracle's outputs."""
    import torch
    c = prefill_inputs(dims, dtype, std, prior, new, kv=kv, gap=gap)
    ref_cache = c.cache.clone()
    idx = np.concatenate([np.arange(c.seq_off[b] + c.prior[b], c.seq_off[b] + c.tot[b])
                          for b in range(len(c.prior))])
    idx_d = torch.as_tensor(idx, device="cuda")
    c.cache[idx_d] = 0
    y = host(c.layer.prefill_step(c.x_dev, c.cu_new, c.prior.astype(np.int32), c.seq_off,
                                  c.cache))
    new_rows, ref_rows = host(c.cache[idx_d]), host(ref_cache[idx_d])
    if kv == "fp8":
        assert np.mean(new_rows == ref_rows) > 0.98
    else:
        assert row_rel_err(new_rows, ref_rows).max() < tol(dtype)
    keep = np.setdiff1d(np.arange(c.cache.shape[0]), idx)
    keep_d = torch.as_tensor(keep, device="cuda")
    assert torch.equal(c.cache[keep_d], ref_cache[keep_d])
    return check_prefill(c, y, query_subset)


def test_prefill_step_v3_fused_in_projection():
    """A query LoRA: the append and the query's first projection share one
    product over [W_kva ; W_qa]."""
    run_step_case(synth.V3, "bf16", 0.02, [0, 21], [24, 9])


@pytest.mark.timeout(300)
def test_prefill_step_v3_large_tiles():
    """670 new tokens: the fused in-projection on the large-tile GEMM, with a
    ragged last row tile; sampled queries."""
    q0 = np.unique(np.concatenate([np.arange(0, 600, 37), np.arange(590, 600)]))
    run_step_case(synth.V3, "bf16", 0.02, [0, 300], [600, 70], gap=3,
                  query_subset=[q0, np.arange(70)])


def test_prefill_step_v2lite():
    """No query LoRA: the append's own product, then the prefill."""
    run_step_case(synth.V2_LITE, "bf16", 0.02, [0, 37, 100], [40, 13, 1])


def test_prefill_step_v3_fp8():
    run_step_case(synth.V3, "bf16", 0.02, [0, 21], [24, 9], kv="fp8")


def test_prefill_step_tiny_f32():
    run_step_case(synth.TINY, "f32", 0.05, [0, 3, 8], [9, 6, 1])
