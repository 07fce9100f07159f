"""Seeded synthetic inputs (weights, hidden states, lengths) for every workload.

This module holds none of the attention arithmetic: it only draws numbers and
rounds them to the storage precision, so that the HIP library and the fp64
oracle can be fed the very same values.  It imports neither of them.

Recipe (stated once, used everywhere):
  * weights: ``numpy.random.default_rng(1234)``; drawn in the fixed order
    W_q | (W_qa, gamma_q, W_qb), W_kva, gamma_kv, W_kvb, W_o, each a row-major
    (out, in) matrix of N(0, std) values (std 0.05 for the tiny fp32 layer,
    0.02 for the DeepSeek-shaped layers); gains are ones, or 1 + 0.1 N(0, 1)
    when ``random_gains`` is set (parity tests use that to prove the gain is
    applied).
  * hidden states: sequence b draws from ``default_rng([1235, b])``, N(0, 1),
    one row per token in position order, so any one sequence can be produced
    without drawing the others.
  * lengths: ``default_rng(1236).integers(lo, hi + 1, B)``.
  * bf16 workloads store every value rounded to bfloat16 (round to nearest,
    ties to even); the arrays returned here are float32 holding exactly those
    values.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_SEED = 1234
HIDDEN_SEED = 1235
LENGTH_SEED = 1236


@dataclass(frozen=True)
class LayerDims:
    hidden: int
    n_heads: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora: int
    q_lora: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    rope_scale: float = 1.0        # YaRN factor; 1 = plain RoPE
    rope_orig_max: int = 4096
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    yarn_mscale: float = 0.0       # YaRN attention-factor coefficient; 0 = none

    @property
    def row(self) -> int:
        return self.kv_lora + self.qk_rope


TINY = LayerDims(hidden=64, n_heads=2, qk_nope=16, qk_rope=8, v_head=16, kv_lora=16)
V2_LITE = LayerDims(hidden=2048, n_heads=16, qk_nope=128, qk_rope=64, v_head=128,
                    kv_lora=512)
V3 = LayerDims(hidden=7168, n_heads=128, qk_nope=128, qk_rope=64, v_head=128,
               kv_lora=512, q_lora=1536)


@dataclass(frozen=True)
class Workload:
    """One benchmark or parity workload, named by what it is."""
    name: str
    dims: LayerDims
    dtype: str                 # "bf16" or "f32": storage precision
    weight_std: float
    kind: str                  # "decode" or "prefill"
    batch: int
    len_lo: int = 0            # decode: cached rows per sequence ~ U{lo..hi}
    len_hi: int = 0
    new_tokens: int = 1        # prefill: new tokens per sequence
    prior: tuple = field(default_factory=tuple)  # prefill: cached rows before
    fixed_lengths: tuple = field(default_factory=tuple)
    kv: str = "dtype"          # latent cache rows: "dtype" or "fp8" (E4M3 + row scale)
    page_rows: int = 0         # > 0: a paged cache, pages handed out in a seeded random order
    q_len: int = 1             # decode: new tokens per sequence and step
    absorb: str = "factored"   # decode weights: "factored" or "materialized" (W^KQ, W^OV)


WORKLOADS = {
    # tiny fp32 layer: 8 cached tokens (positions 0..7) + 1 decode token (pos 8)
    "tiny_f32_decode": Workload("tiny_f32_decode", TINY, "f32", 0.05, "decode", 1,
                                fixed_lengths=(8,)),
    # V2-Lite decode, one sequence with 4096 cached rows, query at position 4096
    "v2lite_decode_b1_s4096": Workload("v2lite_decode_b1_s4096", V2_LITE, "bf16",
                                       0.02, "decode", 1, fixed_lengths=(4096,)),
    # V2-Lite ragged decode, B=64, cached rows ~ U{512..8192}
    "v2lite_decode_b64": Workload("v2lite_decode_b64", V2_LITE, "bf16", 0.02,
                                  "decode", 64, len_lo=512, len_hi=8192),
    # the same batch on an FP8 latent cache (656-byte rows)
    "v2lite_decode_b64_fp8": Workload("v2lite_decode_b64_fp8", V2_LITE, "bf16", 0.02,
                                      "decode", 64, len_lo=512, len_hi=8192, kv="fp8"),
    # the same batch on a paged cache: 64-row pages in a seeded random order
    "v2lite_decode_b64_paged": Workload("v2lite_decode_b64_paged", V2_LITE, "bf16", 0.02,
                                        "decode", 64, len_lo=512, len_hi=8192, page_rows=64),
    # the same batch decoding two new tokens per sequence and step
    "v2lite_decode_b64_q2": Workload("v2lite_decode_b64_q2", V2_LITE, "bf16", 0.02,
                                     "decode", 64, len_lo=512, len_hi=8192, q_len=2),
    # the same batch with materialised absorption (W^KQ, W^OV formed once)
    "v2lite_decode_b64_materialized": Workload("v2lite_decode_b64_materialized", V2_LITE, "bf16",
                                               0.02, "decode", 64, len_lo=512, len_hi=8192,
                                               absorb="materialized"),
    # V3 ragged decode, B=32, cached rows ~ U{2048..16384}
    "v3_decode_b32": Workload("v3_decode_b32", V3, "bf16", 0.02, "decode", 32,
                              len_lo=2048, len_hi=16384),
    # the same batch with materialised absorption
    "v3_decode_b32_materialized": Workload("v3_decode_b32_materialized", V3, "bf16", 0.02,
                                           "decode", 32, len_lo=2048, len_hi=16384,
                                           absorb="materialized"),
    # the same batch on an FP8 latent cache
    "v3_decode_b32_fp8": Workload("v3_decode_b32_fp8", V3, "bf16", 0.02, "decode", 32,
                                  len_lo=2048, len_hi=16384, kv="fp8"),
    # V3 long-context stress: one sequence with 32768 cached rows
    "v3_decode_b1_s32768": Workload("v3_decode_b1_s32768", V3, "bf16", 0.02,
                                    "decode", 1, fixed_lengths=(32768,)),
    # V3 chunked causal prefill: 4 x 4096 new tokens after 0 / 2048 cached
    "v3_prefill_4x4096": Workload("v3_prefill_4x4096", V3, "bf16", 0.02, "prefill",
                                  4, new_tokens=4096, prior=(0, 2048, 0, 2048)),
}


def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32.  Finite inputs only (the synthetic inputs never hold NaN/Inf)."""
    out = np.array(a, dtype=np.float32, copy=True, order="C")
    u = out.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    u += lsb          # cannot wrap for finite values
    u &= np.uint32(0xFFFF0000)
    return out


def to_storage(a, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if dtype == "bf16" else np.ascontiguousarray(a)


def make_weights(dims: LayerDims, std: float, dtype: str, random_gains: bool = False,
                 seed: int = WEIGHT_SEED) -> dict:
    """All layer weights as float32 arrays holding storage-precision values."""
    rng = np.random.default_rng(seed)
    H, dn, dr, dv = dims.n_heads, dims.qk_nope, dims.qk_rope, dims.v_head
    D, dc, dq = dims.hidden, dims.kv_lora, dims.q_lora

    def mat(o, i):
        return to_storage(rng.standard_normal((o, i), dtype=np.float32) * std, dtype)

    def gain(n):
        if random_gains:
            g = 1.0 + 0.1 * rng.standard_normal(n, dtype=np.float32)
        else:
            g = np.ones(n, dtype=np.float32)
        return to_storage(g, dtype)

    w = {}
    if dq:
        w["w_qa"] = mat(dq, D)
        w["q_norm_g"] = gain(dq)
        w["w_qb"] = mat(H * (dn + dr), dq)
    else:
        w["w_q"] = mat(H * (dn + dr), D)
    w["w_kva"] = mat(dc + dr, D)
    w["kv_norm_g"] = gain(dc)
    w["w_kvb"] = mat(H * (dn + dv), dc)
    w["w_o"] = mat(D, H * dv)
    return w


def hidden_states(b: int, n: int, hidden: int, dtype: str, start: int = 0,
                  seed: int = HIDDEN_SEED) -> np.ndarray:
    """Hidden states of sequence b for token positions start .. start+n-1."""
    rng = np.random.default_rng([seed, b])
    if start:
        rng.standard_normal((start, hidden), dtype=np.float32)  # skip earlier tokens
    return to_storage(rng.standard_normal((n, hidden), dtype=np.float32), dtype)


def lengths(w: Workload, seed: int = LENGTH_SEED) -> np.ndarray:
    """Cached rows per sequence (before the new decode token)."""
    if w.fixed_lengths:
        return np.asarray(w.fixed_lengths, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return rng.integers(w.len_lo, w.len_hi + 1, w.batch).astype(np.int64)


def page_table(seq_len, page_rows: int, seed: int = 1237):
    """Block table of a paged cache: every sequence's ceil(len / P) pages
    drawn without replacement from a pool of exactly that many pages, in a
    seeded random order.  Returns (table (B, max_pages) int32, n_pages)."""
    need = (np.asarray(seq_len, dtype=np.int64) + page_rows - 1) // page_rows
    n_pages = int(need.sum())
    perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
    table = np.zeros((len(need), int(need.max())), dtype=np.int32)
    k = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[k:k + m]
        k += m
    return table, n_pages


def decode_layout(lens: np.ndarray, q_len: int = 1):
    """Contiguous per-sequence cache layout for decode: sequence b owns rows
    [seq_off[b], seq_off[b] + lens[b] + q_len) (cached rows plus its new
    tokens)."""
    s = np.asarray(lens, dtype=np.int64) + q_len
    seq_off = np.concatenate([[0], np.cumsum(s)[:-1]]).astype(np.int64)
    return seq_off, s.astype(np.int32), int(s.sum())


def prefill_layout(w: Workload):
    """Cache layout for chunked prefill: sequence b owns rows
    [seq_off[b], seq_off[b] + prior[b] + new_tokens)."""
    prior = np.asarray(w.prior, dtype=np.int64)
    tot = prior + w.new_tokens
    seq_off = np.concatenate([[0], np.cumsum(tot)[:-1]]).astype(np.int64)
    cu_new = np.arange(w.batch + 1, dtype=np.int32) * w.new_tokens
    return seq_off, prior.astype(np.int32), cu_new, int(tot.sum())
