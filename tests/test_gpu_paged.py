"""GPU parity of the paged latent cache (mla_decode_paged,
mla_decode_step_paged), through the C ABI.

The rows of a ragged batch are appended into a contiguous cache by the
library, then copied into a pool of pages in a random order
(oracle.paged.row_index gives each position's pool row).  The paged decode
must give, bit for bit, what the contiguous decode gives on the same rows
(the work split depends on the lengths only, so the arithmetic is the same),
and the outputs are checked against the fp64 oracle at the bf16 / fp32
tolerance."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from oracle import paged as PG
from tests.helpers import DecodeCase, dev, host, row_rel_err, tol
from tests.test_gpu_decode import _compare, chunk

pytestmark = pytest.mark.gpu


def _page_pool(case, page_rows, seed, spare=1.5, shared=None):
    """Copy the contiguous cache of `case` into a pool of pages in random
    order.  shared = (a, b): sequence b's first page is sequence a's."""
    import torch
    lens = case.seq_len
    need = PG.pages_needed(lens, page_rows)
    n_pages = int(need.sum() * spare) + 1
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)
    table = np.full((case.B, int(need.max()) + 1), -1, dtype=np.int32)
    k = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[k:k + m]
        k += m
    if shared is not None:
        a, b = shared
        table[b, 0] = table[a, 0]
    pool = torch.zeros((n_pages * page_rows,) + tuple(case.cache.shape[1:]),
                       dtype=case.cache.dtype, device="cuda")
    for b in range(case.B):
        if shared is not None and b == shared[1]:
            t = np.arange(page_rows, int(lens[b]))  # the shared page is written by its owner
        else:
            t = np.arange(int(lens[b]))
        dst = torch.as_tensor(PG.row_index(table, page_rows, b, t), device="cuda")
        src = torch.as_tensor(int(case.seq_off[b]) + t, device="cuda")
        pool[dst] = case.cache[src]
    torch.cuda.synchronize()
    return pool, table


def _paged_vs_contiguous(case, page_rows, seed, oracle_bs):
    y_c, q_c, o_c = case.run(stages=True)
    pool, table = _page_pool(case, page_rows, seed)
    x = dev(case.x_new, case.layer.torch_dtype)
    y_p, q_p, o_p = case.layer.decode_paged(x, case.seq_len - 1, table, page_rows, case.seq_len,
                                            pool, stages=True)
    assert np.array_equal(host(y_p), host(y_c))
    assert np.array_equal(host(q_p), host(q_c))
    assert np.array_equal(host(o_p), host(o_c))
    y = host(y_p)
    for b in oracle_bs:
        y_ref, _ = case.oracle(b)
        err = row_rel_err(y[b:b + 1], y_ref[None])[0]
        assert err < tol(case.dtype), f"seq {b} (len {case.lens[b]}): y rel err {err:.3e}"


LENS = [0, 1, 14, 31, 32, 33, 63, 64, 65, 130, 700, 1500]


@pytest.mark.parametrize("page_rows", [32, 64, 256])
def test_paged_decode_ring_core(page_rows):
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, LENS)
    _paged_vs_contiguous(case, page_rows, 100 + page_rows, range(len(LENS)))


def test_paged_decode_fp8_ring_core():
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, LENS, kv="fp8")
    _paged_vs_contiguous(case, 64, 7, range(len(LENS)))


def test_paged_decode_generic_core_f32():
    case = DecodeCase(synth.TINY, "f32", 0.05, [0, 1, 7, 31, 32, 100])
    _paged_vs_contiguous(case, 32, 8, range(6))


def test_paged_decode_many_head_core():
    """128 heads (the V3 core), one head group per workgroup wave."""
    case = DecodeCase(synth.V3, "bf16", 0.02, [0, 33, 300, 2100], keep=[0, 3])
    _paged_vs_contiguous(case, 64, 9, [0, 3])


def test_paged_decode_many_head_fp8_core():
    """128 heads on FP8 rows: the raw tiles of the many-head FP8 core come
    through the page list, bit-exact against the contiguous cache."""
    case = DecodeCase(synth.V3, "bf16", 0.02, [0, 33, 300, 2100], keep=[0, 3], kv="fp8")
    _paged_vs_contiguous(case, 64, 10, [0, 3])


def test_paged_decode_shared_prefix_page():
    """Two sequences whose first page is the same pool page read the same
    first rows: equal, bit for bit, to a contiguous cache in which the second
    sequence's first rows are copies of the first's."""
    import torch
    P = 64
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [100, 90, 300], keep=[])
    pool, table = _page_pool(case, P, 10, shared=(0, 1))
    o0, o1 = int(case.seq_off[0]), int(case.seq_off[1])
    case.cache[o1:o1 + P] = case.cache[o0:o0 + P]
    torch.cuda.synchronize()
    y_c = host(case.run())
    x = dev(case.x_new, torch.bfloat16)
    y_p = host(case.layer.decode_paged(x, case.seq_len - 1, table, P, case.seq_len, pool))
    assert np.array_equal(y_p, y_c)


@pytest.mark.parametrize("kv", ["dtype", "fp8"])
def test_paged_decode_step(kv):
    """decode_step_paged writes each new row through the block table (the
    same bytes the contiguous step writes) and returns the contiguous step's
    output; lengths put new rows at the start, middle and end of a page."""
    import torch
    P = 32
    lens = [0, 31, 32, 45, 63, 64, 200]
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, lens, kv=kv)
    pool, table = _page_pool(case, P, 11)
    last_c = torch.as_tensor(case.seq_off + case.seq_len - 1, device="cuda")
    last_p = torch.as_tensor([int(PG.row_index(table, P, b, int(case.seq_len[b]) - 1))
                              for b in range(case.B)], device="cuda")
    pool[last_p] = 0   # the step must write these rows itself
    x = dev(case.x_new, torch.bfloat16)
    y_c = host(case.layer.decode_step(x, case.seq_off, case.seq_len, case.cache))
    y_p = host(case.layer.decode_step_paged(x, table, P, case.seq_len, pool))
    assert torch.equal(pool[last_p], case.cache[last_c])
    assert np.array_equal(y_p, y_c)
    for b in range(case.B):
        y_ref, _ = case.oracle(b)
        assert row_rel_err(y_p[b:b + 1], y_ref[None])[0] < tol("bf16"), b


@pytest.fixture(scope="module")
def paged_b64():
    """The benchmark's 64-sequence batch: contiguous decode, then the same
    rows on 64-row pages in random order; (case, paged host outputs)."""
    w = synth.WORKLOADS["v2lite_decode_b64"]
    case = DecodeCase(w.dims, "bf16", w.weight_std, synth.lengths(w), random_gains=False)
    y_c, q_c, o_c = case.run(stages=True)
    pool, table = _page_pool(case, 64, 12)
    x = dev(case.x_new, case.layer.torch_dtype)
    out = case.layer.decode_paged(x, case.seq_len - 1, table, 64, case.seq_len, pool,
                                  stages=True)
    out = tuple(host(t) for t in out)
    del pool
    return case, out, (host(y_c), host(q_c), host(o_c))


@pytest.mark.timeout(300)
def test_paged_decode_b64_full_size_bit_exact(paged_b64):
    """The paged core run of the timed configuration equals the contiguous
    one bit for bit (y, q_cat, o_lat)."""
    _, out, contig = paged_b64
    for a, b in zip(out, contig):
        assert np.array_equal(a, b)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("part", range(4))
def test_paged_decode_b64_full_size(paged_b64, part):
    """... and every sequence matches the oracle, a quarter per test."""
    case, out, _ = paged_b64
    _compare(case, out, chunk(case.B, part))


def test_paged_decode_large_pages():
    """4096-row pages: a sequence filling exactly one page, one crossing into
    a second, short ones sharing nothing."""
    case = DecodeCase(synth.V2_LITE, "bf16", 0.02, [4095, 4096, 10, 5000], keep=[0, 1, 3])
    _paged_vs_contiguous(case, 4096, 13, [0, 1, 3])


@pytest.mark.parametrize("kv,page_rows", [("dtype", 32), ("dtype", 256), ("fp8", 64)])
def test_paged_prefill_matches_contiguous(kv, page_rows):
    """mla_prefill_paged over a pool of pages in random order gives, bit for
    bit, what mla_prefill gives on the contiguous cache holding the same rows
    (both expand and attend the same rows in the same order), and matches the
    oracle; sequences of several pages with ragged last pages, a long prior
    and a one-token chunk."""
    import types

    import torch
    from tests.test_gpu_prefill import check_prefill, prefill_inputs
    c = prefill_inputs(synth.V2_LITE, "bf16", 0.02, [0, 300, 33], [600, 70, 1], kv=kv)
    prior = c.prior.astype(np.int32)
    y_c = c.layer.prefill(c.x_dev, c.cu_new, prior, c.seq_off, c.cache)
    view = types.SimpleNamespace(seq_len=c.tot, B=len(c.tot), cache=c.cache, seq_off=c.seq_off)
    pool, table = _page_pool(view, page_rows, seed=7)
    y_p = c.layer.prefill_paged(c.x_dev, c.cu_new, prior, table, page_rows, pool)
    assert torch.equal(y_p, y_c)
    check_prefill(c, host(y_p))


def test_paged_prefill_v3():
    """The 128-head layer (query LoRA) over a paged cache, against the oracle."""
    import types

    from tests.test_gpu_prefill import check_prefill, prefill_inputs
    c = prefill_inputs(synth.V3, "bf16", 0.02, [0, 70], [40, 9])
    view = types.SimpleNamespace(seq_len=c.tot, B=len(c.tot), cache=c.cache, seq_off=c.seq_off)
    pool, table = _page_pool(view, 32, seed=3)
    y = c.layer.prefill_paged(c.x_dev, c.cu_new, c.prior.astype(np.int32), table, 32, pool)
    check_prefill(c, host(y))
