"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and its host-side validation returns the documented status
codes (no compute call is made here)."""

import ctypes
import os

import numpy as np
import pytest

from mla_latent_kv_decode_amd import lib as L
from mla_latent_kv_decode_amd import synth


@pytest.fixture(scope="module")
def mla():
    if not os.path.exists(L.LIB_PATH):
        from mla_latent_kv_decode_amd import build
        build.build()
    return L.load()


def cfg(dims=synth.V2_LITE, dtype="bf16", **over):
    c = L.make_config(dims, dtype)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_exports_every_declared_symbol(mla):
    names = L.header_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(mla, n)]
    assert not missing, missing
    assert set(names) == set(L._SIGS), set(names) ^ set(L._SIGS)
    assert mla.mla_abi_version() == 9


def test_status_strings(mla):
    for code in range(0, -7, -1):
        assert mla.mla_status_string(code).decode()
    assert mla.mla_status_string(-99).decode() == "unknown status"


def test_config_check(mla):
    ok = lambda c: mla.mla_config_check(ctypes.byref(c))
    assert ok(cfg()) == L.MLA_OK
    assert ok(cfg(synth.V3)) == L.MLA_OK
    assert ok(cfg(synth.TINY, "f32")) == L.MLA_OK
    assert ok(cfg(qk_rope=7)) == L.MLA_ERR_SHAPE           # RoPE rotates pairs
    assert ok(cfg(qk_rope=0)) == L.MLA_OK                  # no decoupled rope part
    assert ok(cfg(hidden=0)) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(n_heads=-1)) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(q_lora=-1)) == L.MLA_ERR_INVALID_ARG
    c7 = cfg()
    c7.dtype = 7
    assert ok(c7) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(rope_base=0.0)) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(rms_eps=float("nan"))) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(softmax_scale=-1.0)) == L.MLA_ERR_INVALID_ARG
    assert mla.mla_config_check(None) == L.MLA_ERR_INVALID_ARG


def test_yarn_config_check(mla):
    ok = cfg(rope_scale=40.0, rope_orig_max=4096, yarn_beta_fast=32.0, yarn_beta_slow=1.0)
    assert mla.mla_config_check(ctypes.byref(ok)) == L.MLA_OK
    assert mla.mla_config_check(ctypes.byref(cfg(rope_scale=0.0, rope_orig_max=0))) == L.MLA_OK
    assert mla.mla_config_check(ctypes.byref(cfg(rope_scale=40.0, yarn_mscale=0.707))) == L.MLA_OK
    for bad in (dict(rope_scale=4.0, rope_orig_max=0),
                dict(rope_scale=4.0, yarn_beta_fast=1.0, yarn_beta_slow=1.0),
                dict(rope_scale=4.0, yarn_beta_slow=-1.0),
                dict(rope_scale=4.0, yarn_beta_slow=0.0),
                dict(rope_scale=4.0, yarn_mscale=-0.5),
                dict(rope_scale=4.0, yarn_mscale=float("inf")),
                dict(rope_scale=float("nan"))):
        assert mla.mla_config_check(ctypes.byref(cfg(**bad))) == L.MLA_ERR_INVALID_ARG, bad


def test_fp8_cache_config_and_row_bytes(mla):
    """FP8 latent rows: accepted for the shapes the FP8 core serves (bf16
    layer, latent 512, rope 64, a multiple of 16 heads, 128-head layers
    included), refused otherwise; 656 bytes per row (512 codes + 64 bf16 +
    scale, padded to 16)."""
    ok = lambda c: mla.mla_config_check(ctypes.byref(c))
    rb = lambda c: mla.mla_cache_row_bytes(ctypes.byref(c))
    c8 = cfg(kv_storage=L.MLA_KV_FP8_E4M3)
    assert ok(c8) == L.MLA_OK and rb(c8) == 656
    assert rb(cfg()) == 576 * 2 and rb(cfg(synth.TINY, "f32")) == 24 * 4
    assert ok(cfg(kv_storage=2)) == L.MLA_ERR_INVALID_ARG
    assert rb(cfg(kv_storage=2)) == 0
    for bad in (cfg(synth.TINY, "f32", kv_storage=1), cfg(kv_lora=256, kv_storage=1),
                cfg(qk_rope=32, kv_storage=1), cfg(n_heads=24, kv_storage=1)):
        assert ok(bad) == L.MLA_ERR_SHAPE
    assert ok(cfg(n_heads=32, kv_storage=1)) == L.MLA_OK
    assert ok(cfg(synth.V3, kv_storage=1)) == L.MLA_OK


def test_absorb_config(mla):
    """Materialised absorption: accepted for bf16 layers with a 512-wide
    latent (the fused decode path's shapes), refused otherwise; unknown modes
    are invalid."""
    ok = lambda c: mla.mla_config_check(ctypes.byref(c))
    assert ok(cfg(absorb=L.MLA_ABSORB_MATERIALIZED)) == L.MLA_OK
    assert ok(cfg(synth.V3, absorb=L.MLA_ABSORB_MATERIALIZED)) == L.MLA_OK
    assert ok(cfg(absorb=2)) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(absorb=-1)) == L.MLA_ERR_INVALID_ARG
    assert ok(cfg(synth.TINY, "f32", absorb=1)) == L.MLA_ERR_SHAPE
    assert ok(cfg(kv_lora=256, absorb=1)) == L.MLA_ERR_SHAPE


def _i32(a):
    a = np.ascontiguousarray(a, np.int32)
    return a, a.ctypes.data_as(L._I32P)


def _i64(a):
    a = np.ascontiguousarray(a, np.int64)
    return a, a.ctypes.data_as(L._I64P)


def test_append_check(mla):
    c = cfg()

    def chk(pos, slot, rows, T=None):
        pa, pp = _i32(pos)
        sa, sp = _i64(slot)
        return mla.mla_append_check(ctypes.byref(c), pp, sp, len(pa) if T is None else T, rows)

    assert chk([0, 1, 2], [5, 6, 7], 8) == L.MLA_OK
    assert chk([0, 1, 2], [5, 6, 8], 8) == L.MLA_ERR_CAPACITY      # slot == cache_rows
    assert chk([0, 1, 2], [-1, 6, 7], 8) == L.MLA_ERR_CAPACITY
    assert chk([0, 1, 2], [5, 6, 5], 8) == L.MLA_ERR_INVALID_ARG   # duplicate slot
    assert chk([0, -1, 2], [5, 6, 7], 8) == L.MLA_ERR_INVALID_ARG  # negative position
    assert chk([0], [0], 8, T=0) == L.MLA_ERR_INVALID_ARG
    assert chk([0], [0], 0) == L.MLA_ERR_INVALID_ARG
    bad = cfg(qk_rope=3)
    pa, pp = _i32([0])
    sa, sp = _i64([0])
    assert mla.mla_append_check(ctypes.byref(bad), pp, sp, 1, 4) == L.MLA_ERR_SHAPE


def test_decode_check(mla):
    c = cfg()

    def chk(pos, off, ln, rows):
        pa, pp = _i32(pos)
        oa, op = _i64(off)
        la, lp = _i32(ln)
        return mla.mla_decode_check(ctypes.byref(c), pp, op, lp, len(pa), rows)

    assert chk([4, 0], [0, 5], [5, 1], 6) == L.MLA_OK
    assert chk([4, 0], [0, 5], [5, 1], 5) == L.MLA_ERR_CAPACITY    # last row past the end
    assert chk([4, 0], [-1, 5], [5, 1], 6) == L.MLA_ERR_CAPACITY
    assert chk([3, 0], [0, 5], [5, 1], 6) == L.MLA_ERR_INVALID_ARG  # pos != len - 1
    assert chk([4, -1], [0, 5], [5, 0], 6) == L.MLA_ERR_INVALID_ARG  # empty sequence
    assert chk([], [], [], 6) == L.MLA_ERR_INVALID_ARG              # B = 0
    # int64 offsets near the top of the range must not overflow into "fits"
    assert chk([4], [2 ** 62], [5], 2 ** 62) == L.MLA_ERR_CAPACITY


def test_decode_paged_check(mla):
    c = cfg()

    def chk(pos, table, page_rows, ln, rows, writes=0):
        pa, pp = _i32(pos)
        t = np.ascontiguousarray(table, dtype=np.int32)
        ta, tp = _i32(t.reshape(-1))
        la, lp = _i32(ln)
        return mla.mla_decode_paged_check(ctypes.byref(c), pp, tp, t.shape[1], page_rows, lp,
                                          len(pa), rows, writes)

    # 4 pages of 32 rows; sequence 0 (40 rows) on pages 3, 1; sequence 1 (5 rows) on page 0
    ok = ([39, 4], [[3, 1], [0, -7]], 32, [40, 5], 128)
    assert chk(*ok) == L.MLA_OK
    assert chk(*ok, writes=1) == L.MLA_OK
    assert chk([39, 4], [[3, 1], [0, -7]], 32, [40, 5], 127) == L.MLA_ERR_CAPACITY  # page 3 gone
    assert chk([39, 4], [[4, 1], [0, 0]], 32, [40, 5], 128) == L.MLA_ERR_CAPACITY   # page >= 4
    assert chk([39, 4], [[3, -1], [0, 0]], 32, [40, 5], 128) == L.MLA_ERR_CAPACITY  # negative
    assert chk([64, 4], [[3, 1], [0, 0]], 32, [65, 5], 128) == L.MLA_ERR_CAPACITY   # 3 pages > 2
    for bad_p in (16, 48, 0, -32):                                                   # power of 2 >= 32
        assert chk([39, 4], [[3, 1], [0, 0]], bad_p, [40, 5], 128) == L.MLA_ERR_INVALID_ARG
    assert chk([38, 4], [[3, 1], [0, 0]], 32, [40, 5], 128) == L.MLA_ERR_INVALID_ARG  # pos
    # a step writing two new rows onto one cache row (shared last page, same offset)
    assert chk([4, 4], [[2], [2]], 32, [5, 5], 128, writes=1) == L.MLA_ERR_INVALID_ARG
    assert chk([4, 4], [[2], [2]], 32, [5, 5], 128, writes=0) == L.MLA_OK  # reads may share
    # a shared page that a step writes into: sequence 0's new row (position 4,
    # row 68) is a cached row of sequence 1, which would read it overwritten
    assert chk([4, 5], [[2], [2]], 32, [5, 6], 128, writes=1) == L.MLA_ERR_INVALID_ARG
    assert chk([4, 5], [[2], [2]], 32, [5, 6], 128, writes=0) == L.MLA_OK
    # a shared prefix page only read, new rows on each sequence's own page
    assert chk([39, 39], [[2, 3], [2, 1]], 32, [40, 40], 128, writes=1) == L.MLA_OK
    # a sequence naming the same page twice: its new row lands on its own cached row
    assert chk([39], [[2, 2]], 32, [40], 128, writes=1) == L.MLA_ERR_INVALID_ARG


def test_decode_ex_check(mla):
    c = cfg()

    def chk(B, q, ln, off=None, table=None, P=0, rows=1000, append=0):
        args, keep = L.decode_args(B, q, ln, off, table, P, None, append)
        args.cache_rows = rows
        return mla.mla_decode_ex_check(ctypes.byref(c), ctypes.byref(args))

    assert chk(2, 3, [5, 3], off=[0, 10]) == L.MLA_OK
    assert chk(2, 1, [5, 3], off=[0, 10]) == L.MLA_OK
    assert chk(2, 4, [5, 3], off=[0, 10]) == L.MLA_ERR_INVALID_ARG    # seq_len < q_len
    assert chk(2, 0, [5, 3], off=[0, 10]) == L.MLA_ERR_INVALID_ARG    # q_len < 1
    assert chk(2, 17, [50, 30], off=[0, 100]) == L.MLA_ERR_INVALID_ARG  # q_len > 16
    assert chk(2, 16, [50, 30], off=[0, 100]) == L.MLA_OK
    assert chk(2, 2, [5, 3], off=[0, 998]) == L.MLA_ERR_CAPACITY      # past the end
    assert chk(2, 2, [5, 3]) == L.MLA_ERR_INVALID_ARG                 # neither layout
    both = dict(off=[0, 10], table=[[0], [1]], P=32)
    assert chk(2, 2, [5, 3], **both) == L.MLA_ERR_INVALID_ARG         # both layouts
    # paged: 31 pages of 32 rows; the 3 new rows of sequence 0 (positions 30..32)
    # straddle its pages 4 and 9
    assert chk(2, 3, [33, 3], table=[[4, 9], [2, 0]], P=32, rows=1000, append=1) == L.MLA_OK
    assert chk(2, 3, [33, 3], table=[[4, 31], [2, 0]], P=32) == L.MLA_ERR_CAPACITY
    # sequence 1's new rows (positions 0..2 of page 4) collide with sequence 0's
    # position 32 only if both name page 4 at offset 0: position 32 -> page 9
    # offset 0, so pointing sequence 1 at page 9 collides
    assert chk(2, 3, [33, 3], table=[[4, 9], [9, 0]], P=32, append=1) == L.MLA_ERR_INVALID_ARG
    assert chk(2, 3, [33, 3], table=[[4, 9], [9, 0]], P=32, append=0) == L.MLA_OK
    # contiguous ranges that overlap: sequence 0 writes row 4, which sequence 1
    # (rows 3..5) reads as cached; allowed without the append
    assert chk(2, 1, [5, 3], off=[0, 3], append=1) == L.MLA_ERR_INVALID_ARG
    assert chk(2, 1, [5, 3], off=[0, 3], append=0) == L.MLA_OK
    assert chk(2, 1, [5, 3], off=[0, 5], append=1) == L.MLA_OK


def test_prefill_check(mla):
    c = cfg()

    def chk(cu, prior, off, rows):
        ca, cp = _i32(cu)
        pa, pp = _i32(prior)
        oa, op = _i64(off)
        return mla.mla_prefill_check(ctypes.byref(c), cp, pp, op, len(pa), rows)

    assert chk([0, 4, 7], [0, 2], [0, 4], 9) == L.MLA_OK
    assert chk([0, 4, 7], [0, 2], [0, 4], 8) == L.MLA_ERR_CAPACITY
    assert chk([1, 4, 7], [0, 2], [0, 4], 9) == L.MLA_ERR_INVALID_ARG   # cu_new[0] != 0
    assert chk([0, 4, 3], [0, 2], [0, 4], 9) == L.MLA_ERR_INVALID_ARG   # decreasing
    assert chk([0, 4, 7], [0, -2], [0, 4], 9) == L.MLA_ERR_INVALID_ARG
    assert chk([0, 0, 0], [3, 2], [0, 4], 9) == L.MLA_ERR_INVALID_ARG   # no new tokens
    assert chk([0, 4, 7], [2**31 - 3, 0], [0, 0], 2**40) == L.MLA_ERR_INVALID_ARG  # > int32


def test_prefill_step_check(mla):
    """mla_prefill_step writes the new rows itself: they must be distinct cache
    rows, none of them a row some sequence reads as cached; otherwise as
    mla_prefill_check."""
    c = cfg()

    def chk(cu, prior, off, rows):
        ca, cp = _i32(cu)
        pa, pp = _i32(prior)
        oa, op = _i64(off)
        return mla.mla_prefill_step_check(ctypes.byref(c), cp, pp, op, len(pa), rows)

    assert chk([0, 4, 7], [0, 2], [0, 4], 9) == L.MLA_OK
    assert chk([0, 4, 7], [0, 2], [0, 4], 8) == L.MLA_ERR_CAPACITY
    assert chk([0, 4, 7], [0, -2], [0, 4], 9) == L.MLA_ERR_INVALID_ARG
    # sequence 1's new rows 4..6 would overwrite sequence 0's new rows 2..5
    assert chk([0, 4, 7], [0, 0], [2, 4], 9) == L.MLA_ERR_INVALID_ARG
    # sequence 1 (rows 0..4, prior 2) writes rows 2..4, which sequence 0 reads as cached
    assert chk([0, 1, 4], [4, 2], [0, 0], 9) == L.MLA_ERR_INVALID_ARG
    # sequence 0 reads rows 0..2 and writes row 3; sequence 1 writes row 4
    assert chk([0, 1, 2], [3, 0], [0, 4], 9) == L.MLA_OK
    # ... but not at row 3, sequence 0's new row
    assert chk([0, 1, 2], [3, 0], [0, 3], 9) == L.MLA_ERR_INVALID_ARG
    # a shared prefix of 3 rows: both sequences' new rows would start at row 3
    assert chk([0, 2, 4], [3, 3], [0, 0], 16) == L.MLA_ERR_INVALID_ARG


def test_prefill_paged_check(mla):
    """mla_prefill_paged's host checks: the rows it reads (prior + new per
    sequence) must sit on valid pages of the table; the decode checks' page
    size rules."""
    c = cfg()

    def chk(cu, prior, table, page_rows, rows):
        ca, cp = _i32(cu)
        pa, pp = _i32(prior)
        t = np.ascontiguousarray(table, dtype=np.int32)
        ta, tp = _i32(t.reshape(-1))
        return mla.mla_prefill_paged_check(ctypes.byref(c), cp, pp, tp, t.shape[1], page_rows,
                                           len(pa), rows)

    # 4 pages of 32 rows: sequence 0 (2 + 38 rows) on pages 3, 1; sequence 1
    # (0 + 5 rows) on page 0 (its second entry is never read)
    assert chk([0, 38, 43], [2, 0], [[3, 1], [0, -7]], 32, 128) == L.MLA_OK
    assert chk([0, 38, 43], [2, 0], [[3, 4], [0, 0]], 32, 128) == L.MLA_ERR_CAPACITY   # page 4
    assert chk([0, 38, 43], [2, 0], [[3, -1], [0, 0]], 32, 128) == L.MLA_ERR_CAPACITY  # negative
    assert chk([0, 38, 43], [27, 0], [[3, 1], [0, 0]], 32, 128) == L.MLA_ERR_CAPACITY  # 3 pages
    for bad_p in (16, 48, 0):
        assert chk([0, 38, 43], [2, 0], [[3, 1], [0, 0]], bad_p, 128) == L.MLA_ERR_INVALID_ARG
    assert chk([1, 38, 43], [2, 0], [[3, 1], [0, 0]], 32, 128) == L.MLA_ERR_INVALID_ARG
    assert chk([0, 38, 37], [2, 0], [[3, 1], [0, 0]], 32, 128) == L.MLA_ERR_INVALID_ARG
    assert chk([0, 0, 0], [2, 3], [[3, 1], [0, 0]], 32, 128) == L.MLA_ERR_INVALID_ARG
    # pages may be shared (a common prefix read by both sequences)
    assert chk([0, 1, 2], [31, 31], [[2], [2]], 32, 128) == L.MLA_OK


def test_product_path_has_no_oracle_dependency():
    """The package never imports or loads the oracle (test infrastructure
    only), and the binding fails loudly when the library is missing."""
    import re
    pat = re.compile(r"^\s*(from\s+oracle|import\s+oracle)|oracle/", re.M)
    for dirpath, _, files in os.walk(L._PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f
    old = L._lib
    L._lib = None
    try:
        with pytest.raises(RuntimeError):
            L.load(os.path.join(os.path.dirname(L._PKG), "no_such_lib.so"))
    finally:
        L._lib = old


def _plan_invariants(lens, max_parts):
    from mla_latent_kv_decode_amd import lib
    pb, sb, r0, r1 = lib.decode_plan(lens, max_parts)
    P = len(pb) - 1
    assert 1 <= P <= max_parts
    assert pb[0] == 0 and pb[-1] == len(sb) and np.all(np.diff(pb) >= 1)
    assert len(sb) <= len(lens) + max_parts - 1
    # segments in row order cover every row of every sequence exactly once
    nxt = np.zeros(len(lens), np.int64)
    for b, a, e in zip(sb, r0, r1):
        assert a == nxt[b] and a < e <= lens[b]
        assert b == 0 or nxt[b - 1] == lens[b - 1]
        if e < lens[b]:
            assert e % 32 == 0, "cuts inside a sequence fall on tile boundaries"
        nxt[b] = e
    assert np.array_equal(nxt, lens)
    rows = np.array([(r1[pb[p]:pb[p + 1]] - r0[pb[p]:pb[p + 1]]).sum() for p in range(P)])
    return rows, np.diff(pb)


def test_decode_plan_covers_rows_once():
    """Host work list of the split-S core: random ragged batches."""
    rng = np.random.default_rng(7)
    for _ in range(400):
        B = int(rng.integers(1, 80))
        lens = rng.integers(1, int(rng.choice([3, 40, 3000, 40000])), B)
        _plan_invariants(lens, int(rng.integers(1, 600)))


def test_decode_plan_balances_cost():
    """The 64-sequence ragged batch over 256 parts: every part's rows plus its
    per-segment charge is within a tile plus one charge of the mean."""
    from mla_latent_kv_decode_amd import synth
    lens = synth.lengths(synth.WORKLOADS["v2lite_decode_b64"]) + 1
    rows, segs = _plan_invariants(lens, 256)
    assert 240 <= len(rows) <= 256  # the greedy fill may leave a part or two unused
    seg_rows, tile = 64, 32  # the library's per-segment charge and cut alignment
    cost = rows + seg_rows * segs
    assert cost.max() - cost.mean() < tile + seg_rows


def test_decode_plan_tokens_keeps_tail():
    """With q_len new tokens per sequence, each sequence's last segment holds
    at least q_len rows (every token's causal limit lies in it), and the work
    list keeps the invariants of the one-token plan."""
    from mla_latent_kv_decode_amd import lib
    rng = np.random.default_rng(11)
    for _ in range(300):
        q = int(rng.integers(2, 17))
        B = int(rng.integers(1, 70))
        lens = q + rng.integers(0, int(rng.choice([2, 40, 3000, 40000])), B)
        max_parts = int(rng.integers(1, 600))
        _plan_invariants(lens, max_parts)
        pb, sb, r0, r1 = lib.decode_plan(lens, max_parts, q_len=q)
        last = {}
        for b, a, e in zip(sb, r0, r1):
            last[int(b)] = (int(a), int(e))
        assert sorted(last) == list(range(B))
        for b, (a, e) in last.items():
            assert e == lens[b] and e - a >= q, (q, lens[b], a, e)
        nxt = np.zeros(B, np.int64)
        for b, a, e in zip(sb, r0, r1):
            assert a == nxt[b] and a < e
            nxt[b] = e
        assert np.array_equal(nxt, lens)
        assert len(pb) - 1 <= max_parts


def test_decode_plan_tokens_q1_is_plan():
    """q_len = 1 gives mla_decode_plan's work list."""
    import ctypes
    from mla_latent_kv_decode_amd import lib
    L = lib.load()
    lens = np.random.default_rng(12).integers(1, 5000, 40).astype(np.int32)
    P = 64
    outs = []
    for tok in (False, True):
        pb = np.zeros(P + 1, np.int32)
        sb, r0, r1 = (np.zeros(40 + P - 1, np.int32) for _ in range(3))
        n_p, n_s = ctypes.c_int32(), ctypes.c_int32()
        ptr = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        args = (ptr(pb), ptr(sb), ptr(r0), ptr(r1), ctypes.byref(n_p), ctypes.byref(n_s))
        rc = (L.mla_decode_plan_tokens(40, ptr(lens), 1, P, *args) if tok
              else L.mla_decode_plan(40, ptr(lens), P, *args))
        assert rc == 0
        outs.append((pb[:n_p.value + 1].copy(), sb[:n_s.value].copy(), r0[:n_s.value].copy(),
                     r1[:n_s.value].copy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_decode_plan_errors():
    from mla_latent_kv_decode_amd import lib
    with pytest.raises(lib.MLAError):
        lib.decode_plan([5, 0, 3], 8)
    with pytest.raises(lib.MLAError):
        lib.decode_plan([5], 0)
    with pytest.raises(lib.MLAError):
        lib.decode_plan([5, 3], 8, q_len=4)   # a length below q_len
    with pytest.raises(lib.MLAError):
        lib.decode_plan([50], 8, q_len=17)    # beyond the largest q_len
