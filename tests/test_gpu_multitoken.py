"""GPU parity of multi-token decode (mla_decode_ex with q_len new tokens per
sequence), through the C ABI.

Sequence b holds lens[b] cached rows plus its q_len new tokens' rows
(appended through the library: write, then read).  New token j sits at
position lens[b] + j and sees positions 0 .. lens[b] + j (the offset causal
mask).  The fp64 oracle runs the same step (oracle.mla.mla_step with the
q_len new tokens of the sequence at once); outputs to the bf16 / fp32
tolerance, max relative error per output row."""

import numpy as np
import pytest

from mla_latent_kv_decode_amd import synth
from oracle import fp8 as F8
from oracle import mla as O
from oracle import paged as PG
from tests.helpers import dev, fill_sequence, host, make_layer, oracle_shape, row_rel_err, tol

pytestmark = pytest.mark.gpu


class MTCase:
    def __init__(self, dims, dtype, std, lens, q_len, kv="dtype", keep=None):
        import torch
        self.dims, self.dtype, self.kv, self.q = dims, dtype, kv, q_len
        self.lens = np.asarray(lens, dtype=np.int64)
        self.B = len(lens)
        self.w = synth.make_weights(dims, std, dtype, random_gains=True)
        self.layer = make_layer(dims, dtype, self.w, kv)
        self.seq_len = (self.lens + q_len).astype(np.int32)
        self.seq_off = np.concatenate([[0], np.cumsum(self.seq_len)[:-1]]).astype(np.int64)
        self.cache = self.layer.new_cache(int(self.seq_len.sum()))
        keep = set(range(self.B)) if keep is None else set(keep)
        self.hidden, x_new = {}, []
        for b in range(self.B):
            x, _ = fill_sequence(self.layer, dims, dtype, b, int(self.seq_len[b]), self.cache,
                                 int(self.seq_off[b]), keep=True)
            if b in keep:
                self.hidden[b] = x
            x_new.append(x[-q_len:])
        self.x_new = np.concatenate(x_new)
        torch.cuda.synchronize()

    def x(self):
        return dev(self.x_new, self.layer.torch_dtype)

    def run(self, **kw):
        return host(self.layer.decode_ex(self.x(), self.seq_len, self.cache, q_len=self.q,
                                         seq_off=self.seq_off, **kw))

    def oracle(self, b):
        shp = oracle_shape(self.dims)
        L, xb = int(self.lens[b]), self.hidden[b]
        prior = (O.latent_rows(xb[:L], np.arange(L), self.w["w_kva"], self.w["kv_norm_g"], shp)
                 if L else np.zeros((0, shp.row)))
        store = (lambda r: F8.fp8_rows(r, shp.kv_lora)) if self.kv == "fp8" else None
        return O.mla_step(xb[L:L + self.q], np.arange(L, L + self.q), prior, self.w, shp,
                          kv_store=store)["y"]

    def check(self, y, bs=None):
        for b in (range(self.B) if bs is None else bs):
            ref = self.oracle(b)
            got = y[b * self.q:(b + 1) * self.q]
            err = row_rel_err(got, ref).max()
            assert err < tol(self.dtype), f"seq {b} (len {self.lens[b]}): rel err {err:.3e}"


LENS = [0, 1, 14, 30, 31, 32, 33, 63, 100, 700, 1500]


@pytest.mark.parametrize("q_len", [2, 4])
def test_multitoken_ring_core(q_len):
    case = MTCase(synth.V2_LITE, "bf16", 0.02, LENS, q_len)
    case.check(case.run())


def test_multitoken_q1_is_decode():
    """q_len = 1 through mla_decode_ex is mla_decode, bit for bit."""
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [0, 31, 700], 1, keep=[])
    y_ex = case.run()
    y = host(case.layer.decode(case.x(), case.seq_len - 1, case.seq_off, case.seq_len,
                               case.cache))
    assert np.array_equal(y_ex, y)


def test_multitoken_fp8_ring_core():
    case = MTCase(synth.V2_LITE, "bf16", 0.02, LENS, 3, kv="fp8")
    case.check(case.run())


def test_multitoken_generic_core_f32():
    case = MTCase(synth.TINY, "f32", 0.05, [0, 1, 7, 31, 32, 100], 3)
    case.check(case.run())


def test_multitoken_many_head_core():
    case = MTCase(synth.V3, "bf16", 0.02, [0, 33, 300, 2100], 2, keep=[0, 3])
    case.check(case.run(), [0, 3])


def test_multitoken_many_head_fp8_core():
    case = MTCase(synth.V3, "bf16", 0.02, [0, 33, 300, 2100], 2, keep=[0, 3], kv="fp8")
    case.check(case.run(), [0, 3])


def test_multitoken_paged_and_append():
    """Paged cache (64-row pages in random order) with the append of the new
    rows: the rows it writes and its outputs equal, bit for bit, those of the
    same call on the contiguous cache (the step's projection sums in its own
    order, so rows are compared with the step's, not with the bulk append's);
    outputs against the oracle."""
    import torch
    P, q = 64, 3
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [0, 61, 62, 64, 200, 1000], q)
    need = PG.pages_needed(case.seq_len, P)
    perm = np.random.default_rng(3).permutation(int(need.sum()) + 5)
    table = np.zeros((case.B, int(need.max())), dtype=np.int32)
    k = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[k:k + m]
        k += m
    pool = case.layer.new_cache((int(need.sum()) + 5) * P)
    new_p, new_c = [], []
    for b in range(case.B):
        t = np.arange(int(case.seq_len[b]))
        dst = torch.as_tensor(PG.row_index(table, P, b, t), device="cuda")
        src = torch.as_tensor(int(case.seq_off[b]) + t, device="cuda")
        pool[dst] = case.cache[src]
        new_p.append(PG.row_index(table, P, b, t[-q:]))
        new_c.append(int(case.seq_off[b]) + t[-q:])
    new_p = torch.as_tensor(np.concatenate(new_p), device="cuda")
    new_c = torch.as_tensor(np.concatenate(new_c), device="cuda")
    pool[new_p] = 0        # both calls must write these rows themselves
    case.cache[new_c] = 0
    y_c = case.run(append=True)
    y_p = host(case.layer.decode_ex(case.x(), case.seq_len, pool, q_len=q, block_table=table,
                                    page_rows=P, append=True))
    assert torch.equal(pool[new_p], case.cache[new_c])
    assert bool(case.cache[new_c].abs().sum() > 0)
    assert np.array_equal(y_p, y_c)
    case.check(y_p)


def test_multitoken_long_sequences_split():
    """Sequences long enough to be cut into several segments (one partial
    per segment and token, merged by the combine); the planner keeps at
    least q_len rows in each sequence's last segment."""
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [4095, 4096, 4097, 8190, 33], 4, keep=[0, 3, 4])
    case.check(case.run(), [0, 3, 4])


def test_multitoken_max_q_len():
    """q_len = 16, the largest allowed: sequences with no earlier rows (all
    16 rows are new tokens) and longer ones."""
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [0, 1, 15, 16, 17, 300], 16)
    case.check(case.run())


def test_multitoken_fp8_paged_append():
    """FP8 rows, 32-row pages in random order, two new tokens appended by the
    call: the rows written and the outputs equal the contiguous call's, and
    the outputs match the oracle reading its quantised rows."""
    import torch
    P, q = 32, 2
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [0, 30, 31, 32, 95, 400], q, kv="fp8")
    need = PG.pages_needed(case.seq_len, P)
    perm = np.random.default_rng(4).permutation(int(need.sum()))
    table = np.zeros((case.B, int(need.max())), dtype=np.int32)
    k = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[k:k + m]
        k += m
    pool = case.layer.new_cache(int(need.sum()) * P)
    new_p, new_c = [], []
    for b in range(case.B):
        t = np.arange(int(case.seq_len[b]))
        pool[torch.as_tensor(PG.row_index(table, P, b, t), device="cuda")] = \
            case.cache[torch.as_tensor(int(case.seq_off[b]) + t, device="cuda")]
        new_p.append(PG.row_index(table, P, b, t[-q:]))
        new_c.append(int(case.seq_off[b]) + t[-q:])
    new_p = torch.as_tensor(np.concatenate(new_p), device="cuda")
    new_c = torch.as_tensor(np.concatenate(new_c), device="cuda")
    pool[new_p] = 0
    case.cache[new_c] = 0
    y_c = case.run(append=True)
    y_p = host(case.layer.decode_ex(case.x(), case.seq_len, pool, q_len=q, block_table=table,
                                    page_rows=P, append=True))
    assert torch.equal(pool[new_p], case.cache[new_c])
    assert np.array_equal(y_p, y_c)
    case.check(y_p)


def test_multitoken_generic_core_f32_append():
    """The fp32 build's generic path with the append: the call writes the
    q_len new rows itself (zeroed first) and matches the oracle."""
    import torch
    q = 3
    case = MTCase(synth.TINY, "f32", 0.05, [0, 1, 7, 40], q)
    new = torch.as_tensor(np.concatenate([int(case.seq_off[b]) + np.arange(int(case.seq_len[b]) - q,
                                                                           int(case.seq_len[b]))
                                          for b in range(case.B)]), device="cuda")
    case.cache[new] = 0
    y = case.run(append=True)
    assert bool(case.cache[new].abs().sum() > 0)
    case.check(y)


@pytest.mark.parametrize("kv", ["dtype", "fp8"])
def test_multitoken_paged_is_deterministic(kv):
    """Three runs of the same two-token paged decode give the same bits (the
    partials of a sequence are merged in slot order, independent of timing)."""
    P, q = 64, 2
    case = MTCase(synth.V2_LITE, "bf16", 0.02, [10, 700, 3000, 5000, 64], q, kv=kv, keep=[])
    import torch
    need = PG.pages_needed(case.seq_len, P)
    table = np.zeros((case.B, int(need.max())), dtype=np.int32)
    perm = np.random.default_rng(5).permutation(int(need.sum()))
    k = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[k:k + m]
        k += m
    pool = case.layer.new_cache(int(need.sum()) * P)
    for b in range(case.B):
        t = np.arange(int(case.seq_len[b]))
        pool[torch.as_tensor(PG.row_index(table, P, b, t), device="cuda")] = \
            case.cache[torch.as_tensor(int(case.seq_off[b]) + t, device="cuda")]
    runs = [host(case.layer.decode_ex(case.x(), case.seq_len, pool, q_len=q, block_table=table,
                                      page_rows=P)) for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])
    assert np.all(np.isfinite(runs[0]))


def test_multitoken_token_pairs_two_head_groups():
    """32 heads (two 16-head groups) and two new tokens: the paired query
    tile takes its second token's rows H rows further on in q_cat."""
    import dataclasses
    dims = dataclasses.replace(synth.V2_LITE, n_heads=32)
    case = MTCase(dims, "bf16", 0.02, [0, 31, 700, 2000], 2)
    case.check(case.run())
