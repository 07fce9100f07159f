"""Shared set-up for the GPU parity tests: seeded weights and hidden states
(from ``synth``), caches filled through the library's own append, and the fp64
oracle evaluated on the very same inputs."""

from __future__ import annotations

import numpy as np

from mla_latent_kv_decode_amd import synth
from oracle import fp8 as F8
from oracle import mla as O

APPEND_CHUNK = 8192


def oracle_shape(d: synth.LayerDims) -> O.MLAShape:
    return O.MLAShape(hidden=d.hidden, n_heads=d.n_heads, qk_nope=d.qk_nope, qk_rope=d.qk_rope,
                      v_head=d.v_head, kv_lora=d.kv_lora, q_lora=d.q_lora,
                      rope_base=d.rope_base, rms_eps=d.rms_eps, rope_scale=d.rope_scale,
                      rope_orig_max=d.rope_orig_max, yarn_beta_fast=d.yarn_beta_fast,
                      yarn_beta_slow=d.yarn_beta_slow, yarn_mscale=d.yarn_mscale)


def tol(dtype: str) -> float:
    """Max relative error per output row (max|g - r| / max|r|): 1e-2 for bf16
    storage with fp32 accumulation, 1e-4 for the fp32 build."""
    return 1e-2 if dtype == "bf16" else 1e-4


def row_rel_err(g, r) -> np.ndarray:
    g = np.asarray(g, np.float64).reshape(len(g), -1)
    r = np.asarray(r, np.float64).reshape(len(r), -1)
    return np.max(np.abs(g - r), axis=1) / np.maximum(np.max(np.abs(r), axis=1), 1e-30)


def dev(a, torch_dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch_dtype)


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def make_layer(dims, dtype, weights, kv="dtype", absorb="factored"):
    import torch
    from mla_latent_kv_decode_amd.lib import MLALayer
    layer = MLALayer(dims, dtype, kv=kv, absorb=absorb)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    layer.absorb_weights({k: dev(v, tdt) for k, v in weights.items()})
    return layer


def fill_sequence(layer, dims, dtype, b, n_tokens, cache, base_slot, keep=False):
    """Append tokens 0..n_tokens-1 of sequence b (hidden states from synth) into
    cache rows base_slot + i; returns the hidden states if ``keep``."""
    tdt = layer.torch_dtype
    kept = []
    x = None
    for s in range(0, n_tokens, APPEND_CHUNK):
        n = min(APPEND_CHUNK, n_tokens - s)
        x = synth.hidden_states(b, n, dims.hidden, dtype, start=s)
        layer.append(dev(x, tdt), np.arange(s, s + n), base_slot + np.arange(s, s + n), cache)
        if keep:
            kept.append(x)
    return (np.concatenate(kept) if keep else None), x[-1]


class DecodeCase:
    """A ragged decode batch: sequence b has lens[b] cached rows, appended
    through the library, and one new token at position lens[b] (also appended
    first: write, then read through the new position)."""

    def __init__(self, dims, dtype, std, lens, random_gains=True, keep=None, layer=None,
                 weights=None, kv="dtype", absorb="factored"):
        import torch
        self.dims, self.dtype, self.kv = dims, dtype, kv
        self.lens = np.asarray(lens, dtype=np.int64)
        self.B = len(self.lens)
        self.w = weights if weights is not None else synth.make_weights(
            dims, std, dtype, random_gains=random_gains)
        self.layer = layer if layer is not None else make_layer(dims, dtype, self.w, kv, absorb)
        self.seq_off, self.seq_len, self.total = synth.decode_layout(self.lens)
        self.cache = self.layer.new_cache(self.total)
        keep = set(range(self.B)) if keep is None else set(keep)
        self.hidden = {}
        last = []
        for b in range(self.B):
            x, xl = fill_sequence(self.layer, dims, dtype, b, int(self.lens[b]) + 1, self.cache,
                                  int(self.seq_off[b]), keep=b in keep)
            if b in keep:
                self.hidden[b] = x
            last.append(xl)
        self.x_new = np.stack(last)
        torch.cuda.synchronize()

    def run(self, stages=False):
        x = dev(self.x_new, self.layer.torch_dtype)
        return self.layer.decode(x, self.seq_len - 1, self.seq_off, self.seq_len, self.cache,
                                 stages=stages)

    def oracle(self, b, absorbed_only=False):
        """(y of the non-absorbed fp64 step, the absorbed step's dict) for
        sequence b; with absorbed_only, y comes from the absorbed form (pinned
        equal to the non-absorbed one) and the K/V expansion is skipped."""
        shp = oracle_shape(self.dims)
        L = int(self.lens[b])
        xb = self.hidden[b]
        rows_prior = (O.latent_rows(xb[:L], np.arange(L), self.w["w_kva"], self.w["kv_norm_g"],
                                    shp) if L else np.zeros((0, shp.row)))
        store = (lambda r: F8.fp8_rows(r, shp.kv_lora)) if self.kv == "fp8" else None
        if absorbed_only:
            rows = np.concatenate([rows_prior, O.latent_rows(
                xb[L:L + 1], np.array([L]), self.w["w_kva"], self.w["kv_norm_g"], shp)])
        else:
            r = O.mla_step(xb[L:L + 1], np.array([L]), rows_prior, self.w, shp, kv_store=store)
            rows = np.concatenate([rows_prior, r["rows_new"]])
        if store is not None:
            rows = store(rows)
        a = O.absorbed_step(xb[L:L + 1], np.array([L]), rows, self.w, shp)
        return (a["y"][0] if absorbed_only else r["y"][0]), a
