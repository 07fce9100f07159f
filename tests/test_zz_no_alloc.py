"""mla_decode_step_noalloc: the decode step whose workspace is the library's
static device scratch, called through the C ABI, against mla_decode_step
(same kernels, same work split: bit for bit) and against the fp64 oracle at
the bf16 tolerance, on two calls in a row (the second smaller); plus its
refusals (a batch beyond the static scratch, a stream being captured)."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from tests.helpers import DecodeCase, dev, host, row_rel_err, tol

pytestmark = pytest.mark.gpu


def _step_both(case):
    """(y of mla_decode_step, y of mla_decode_step_noalloc, new rows of
    each) on the same inputs; the new rows are wiped before each call so
    that each call writes them itself."""
    import torch
    last = torch.as_tensor(case.seq_off + case.seq_len - 1, device="cuda")
    x = dev(case.x_new, torch.bfloat16)
    case.cache[last] = 0
    y_ws = case.layer.decode_step(x, case.seq_off, case.seq_len, case.cache).clone()
    rows_ws = case.cache[last].clone()
    case.cache[last] = 0
    y_na = case.layer.decode_step_noalloc(x, case.seq_off, case.seq_len, case.cache)
    rows_na = case.cache[last].clone()
    torch.cuda.synchronize()
    return y_ws, y_na, rows_ws, rows_na


def _check_case(case):
    import torch
    y_ws, y_na, rows_ws, rows_na = _step_both(case)
    assert torch.equal(rows_na.view(torch.int16), rows_ws.view(torch.int16))
    assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
    y = host(y_na)
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol("bf16"), f"seq {b} (len {case.lens[b]}): y rel err {err:.3e}"


def test_noalloc_step_matches_workspace_step_twice():
    """A 24-sequence batch, then a smaller 5-sequence batch with other lengths
    on the same handle: the static scratch keeps the first call's contents,
    which the second must not see."""
    lens_a = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200, 700, 1500, 3000, 40, 5, 900, 2048,
              128, 129, 511, 512, 4000]
    a = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens_a)
    _check_case(a)
    b = DecodeCase(synth.V2_LITE, "bf16", 0.02, [2500, 3, 64, 777, 10], layer=a.layer,
                   weights=a.w)
    _check_case(b)


def test_noalloc_refuses_batch_beyond_scratch():
    """2,000 one-row sequences need ~75 MB of split partials: refused with
    MLA_ERR_WORKSPACE before anything is launched (the cache is untouched)."""
    import torch
    from mla_latent_kv_decode_amd.lib import MLAError, MLA_ERR_WORKSPACE
    d = synth.V2_LITE
    w = synth.make_weights(d, 0.02, "bf16")
    from tests.helpers import make_layer
    layer = make_layer(d, "bf16", w)
    B = 2000
    cache = torch.full((B, d.row), 3.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((B, d.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MLAError) as e:
        layer.decode_step_noalloc(x, np.arange(B), np.ones(B, np.int32), cache)
    assert e.value.status == MLA_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((cache == 3.0).all())


def test_noalloc_refuses_graph_capture():
    """While the handle's stream is being captured the call returns
    MLA_ERR_STATE and records nothing."""
    import torch
    from mla_latent_kv_decode_amd.lib import MLAError, MLA_ERR_STATE
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [10, 20], keep=[])
    x = dev(case.x_new, torch.bfloat16)
    out = torch.empty((case.B, synth.V2_LITE.hidden), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    caught = []
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            try:
                case.layer.decode_step_noalloc(x, case.seq_off, case.seq_len, case.cache, out=out)
            except MLAError as e:
                caught.append(e.status)
    torch.cuda.synchronize()
    assert caught == [MLA_ERR_STATE]
