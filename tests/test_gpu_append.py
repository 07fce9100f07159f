"""GPU tests of the latent-cache append: slot indexing is bit-exact (sentinel
rows stay untouched, raw scatter copies bits), appended rows match the oracle's
[RMSNorm(c) | RoPE(k_rope)], and host-side errors leave the cache untouched."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import lib as L
from mla_latent_kv_decode_amd import synth
from oracle import mla as O
from tests.helpers import dev, host, make_layer, oracle_shape, row_rel_err, tol

pytestmark = pytest.mark.gpu

SENTINEL = 0xFFC1  # a bf16 NaN pattern no computation produces


def _sentinel_cache(rows, width):
    import torch
    return torch.full((rows, width), SENTINEL - 65536, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("dims,T", [(synth.V2_LITE, 300), (synth.V3, 300),
                                    (synth.V2_LITE, 7000), (synth.V3, 4500)])
def test_append_rows_and_indexing(dims, T):
    """T = 300 takes the split-K tile GEMM for the kv_a projection; 7000 and
    4500 rows (not multiples of the 256-row tile) take the large-tile GEMM."""
    import torch
    w = synth.make_weights(dims, 0.02, "bf16", random_gains=True)
    layer = make_layer(dims, "bf16", w)
    rows = max(5000, 2 * T)
    rng = np.random.default_rng(11)
    slot = rng.choice(rows, size=T, replace=False).astype(np.int64)
    pos = rng.integers(0, 40000, size=T).astype(np.int32)
    x = synth.hidden_states(3, T, dims.hidden, "bf16")
    cache = _sentinel_cache(rows, dims.row)
    layer.append(dev(x, torch.bfloat16), pos, slot, cache)
    torch.cuda.synchronize()
    bits = cache.view(torch.int16).cpu().numpy().astype(np.uint16)
    untouched = np.setdiff1d(np.arange(rows), slot)
    assert np.all(bits[untouched] == SENTINEL)
    got = host(cache)[slot]
    ref = O.latent_rows(x, pos, w["w_kva"], w["kv_norm_g"], oracle_shape(dims))
    err = row_rel_err(got, ref)
    assert err.max() < tol("bf16"), err.max()


def test_cache_write_is_bit_exact():
    import torch
    dims = synth.V2_LITE
    layer = make_layer(dims, "bf16", synth.make_weights(dims, 0.02, "bf16"))
    rows, T = 3000, 777
    rng = np.random.default_rng(12)
    slot = rng.permutation(rows)[:T].astype(np.int64)
    src = torch.from_numpy(rng.integers(-32768, 32767, size=(T, dims.row),
                                        dtype=np.int16)).cuda()
    cache = _sentinel_cache(rows, dims.row)
    layer.cache_write(src.view(torch.bfloat16), slot, cache)
    torch.cuda.synchronize()
    got = cache.view(torch.int16).cpu().numpy()
    assert np.array_equal(got[slot], src.cpu().numpy())
    rest = np.setdiff1d(np.arange(rows), slot)
    assert np.all(got[rest].astype(np.uint16) == SENTINEL)


def test_errors_leave_cache_untouched():
    import torch
    dims = synth.V2_LITE
    w = synth.make_weights(dims, 0.02, "bf16")
    layer = L.MLALayer(dims, "bf16")
    x = dev(synth.hidden_states(0, 4, dims.hidden, "bf16"), torch.bfloat16)
    cache = _sentinel_cache(16, dims.row)
    with pytest.raises(L.MLAError) as e:      # append before the weights are absorbed
        layer.append(x, [0, 1, 2, 3], [0, 1, 2, 3], cache)
    assert e.value.status == L.MLA_ERR_STATE
    layer.absorb_weights({k: dev(v, torch.bfloat16) for k, v in w.items()})
    with pytest.raises(L.MLAError) as e:      # slot == cache_rows
        layer.append(x, [0, 1, 2, 3], [0, 1, 2, 16], cache)
    assert e.value.status == L.MLA_ERR_CAPACITY
    with pytest.raises(L.MLAError) as e:      # duplicate slot
        layer.append(x, [0, 1, 2, 3], [0, 1, 2, 2], cache)
    assert e.value.status == L.MLA_ERR_INVALID_ARG
    with pytest.raises(L.MLAError) as e:      # decode: sequence past the cache end
        layer.decode(x[:1], [9], [10], [10], cache)
    assert e.value.status == L.MLA_ERR_CAPACITY
    torch.cuda.synchronize()
    assert np.all(cache.view(torch.int16).cpu().numpy().astype(np.uint16) == SENTINEL)
