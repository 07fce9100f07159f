"""fp64 NumPy oracle: Multi-Head Latent Attention, non-absorbed form.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is float64;
nothing here rounds to bf16.  Matrices are row-major ``(out, in)`` like a
linear layer's weight, so ``y = x @ W.T``.

Notation (row-major, one row per token):
  D  hidden size            H   heads
  dn qk_nope (per head)     dr  qk_rope (per head query, shared key)
  dv v_head                 dc  kv_lora_rank (latent width)
  dq q_lora_rank (0 = the query is projected directly from the hidden state)
  R = dc + dr               one cached latent row: [c_kv | k_rope]

Readings of the pages where they are silent or garbled:
  * RMSNorm is the textbook x / sqrt(mean(x^2) + eps) * gamma; eps = 1e-6.
    It is applied to the dc latent entries only; k_rope gets RoPE only.
  * RoPE rotates adjacent pairs (2i, 2i+1) as complex numbers by
    pos * base^(-2i/d); positions are 0-based; the i-th cached row of a
    sequence has position i.
  * Per-head row layouts: q_proj rows are [q_nope_h (dn) | q_rope_h (dr)] per
    head; kv_b_proj rows are [K_nope_h (dn) ; V_h (dv)] per head.
  * The softmax scale is 1/sqrt(dn + dr) (times YaRN's attention factor
    under context extension, see yarn_attention_factor).
  * A query at position p sees cache rows 0..p of its own sequence (the new
    rows are written to the cache before it is read).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F64 = np.float64


@dataclass(frozen=True)
class MLAShape:
    """Layer dimensions, following the layer constructor of the MLA post
    ("Multi-Head Latent Attention", section 3.2 Code) extended with the
    decoupled-RoPE widths of section 3.6 and the query LoRA of section 3.1."""

    hidden: int
    n_heads: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora: int
    q_lora: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(qk_nope + qk_rope)
    # YaRN context extension of RoPE (see rope_theta): factor 1 = plain RoPE
    rope_scale: float = 1.0
    rope_orig_max: int = 4096
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    yarn_mscale: float = 0.0   # m of yarn_attention_factor; 0 = softmax scale unchanged

    @property
    def theta(self) -> np.ndarray:
        return rope_theta(self.qk_rope, self.rope_base, self.rope_scale, self.rope_orig_max,
                          self.yarn_beta_fast, self.yarn_beta_slow)

    @property
    def row(self) -> int:
        return self.kv_lora + self.qk_rope

    @property
    def scale(self) -> float:
        if self.softmax_scale:
            return float(self.softmax_scale)
        return (yarn_attention_factor(self.rope_scale, self.yarn_mscale)
                / np.sqrt(self.qk_nope + self.qk_rope))


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def rms_norm(a, gamma, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times the gain.

    The C-engine notes ("Deepseek V2 Lite Inference Engine in C", base
    operations) name RMSNorm; the MLA post (section 3.5 Code, ``norm_ckv`` /
    ``norm_cq``) applies it to the compressed vectors.  Textbook form.
    """
    a = _f64(a)
    ms = np.mean(a * a, axis=-1, keepdims=True)
    return a / np.sqrt(ms + eps) * _f64(gamma)


def yarn_pair_at(turns: float, d: int, base: float, orig_max: int) -> float:
    """The (fractional) pair index i at which pair i of plain RoPE turns
    ``turns`` times over ``orig_max`` positions: orig_max * base^(-2i/d) /
    (2 pi) = turns, solved for i."""
    return d * np.log(orig_max / (2.0 * np.pi * turns)) / (2.0 * np.log(base))


def rope_theta(d: int, base: float, scale: float = 1.0, orig_max: int = 4096,
               beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Per-pair rotation frequencies theta_i (i < d / 2).

    Plain RoPE (MLA post, section 3.7): theta_i = base^(-2i/d).  With a
    context-extension factor scale = s > 1: YaRN, which the C-engine notes
    ("Deepseek V2 Lite Inference Engine in C", Todos and base operations) name
    without a formula.  Reading: YaRN's "NTK-by-parts" interpolation in the
    form DeepSeek's layers run it.  Pairs that turn more than beta_fast times
    over the original context keep theta_i, pairs that turn fewer than
    beta_slow times are slowed to theta_i / s, and the band in between blends
    the two with a weight that is linear in the PAIR INDEX: the band runs from
    lo = floor(pair index where a pair turns beta_fast times) to hi =
    ceil(pair index where it turns beta_slow times), both clamped to
    [0, d/2 - 1] (hi raised to lo + 0.001 when they meet);
    w_i = clip((i - lo) / (hi - lo), 0, 1) and theta'_i = (1 - w_i) theta_i +
    w_i theta_i / s.
    """
    theta = base ** (-np.arange(0, d, 2, dtype=F64) / d)
    if scale <= 1.0:
        return theta
    half = d // 2
    lo = max(float(np.floor(yarn_pair_at(beta_fast, d, base, orig_max))), 0.0)
    hi = min(float(np.ceil(yarn_pair_at(beta_slow, d, base, orig_max))), float(half - 1))
    if hi <= lo:
        hi = lo + 0.001
    w = np.clip((np.arange(half, dtype=F64) - lo) / (hi - lo), 0.0, 1.0)
    return (1.0 - w) * theta + w * theta / scale


def yarn_attention_factor(scale: float, mscale: float) -> float:
    """Multiplier of the softmax scale under YaRN context extension.

    The published YaRN method sharpens the logits by a temperature with
    sqrt(1/t) = 0.1 ln(s) + 1; DeepSeek's layers weight the logarithm by a
    per-model coefficient m (0 = no change) and multiply the softmax scale by
    (0.1 m ln(s) + 1)^2.  Factor 1 for s <= 1."""
    if scale <= 1.0:
        return 1.0
    return float((0.1 * mscale * np.log(scale) + 1.0) ** 2)


def rope(x, pos, base: float, theta=None) -> np.ndarray:
    """Rotary position embedding on the last axis.

    MLA post, section 3.7 Code (``RoPE`` / ``apply_rope``): pair i of the last
    axis, (x[2i], x[2i+1]), is read as the complex number x[2i] + j x[2i+1] and
    multiplied by exp(j * pos * theta_i) with theta_i = base^(-2i/d), d even
    (or the given per-pair frequencies ``theta``, e.g. from ``rope_theta``).
    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = _f64(x)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    if theta is None:
        theta = base ** (-np.arange(0, d, 2, dtype=F64) / d)
    theta = _f64(theta)
    ang = _f64(pos)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    u, v = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=F64)
    out[..., 0::2] = u * cos - v * sin
    out[..., 1::2] = u * sin + v * cos
    return out


def latent_rows(x, pos, w_kva, kv_norm_g, shape: MLAShape) -> np.ndarray:
    """The cached row of each token: [RMSNorm(c_kv) | RoPE(k_rope)].

    The down-projection kv_a_proj produces the latent and the shared RoPE key
    in one matrix ("Deepseek V2 Lite Inference Engine in C", MLA notes: kv_a_proj
    fuses the KV down-projection and the shared RoPE key); the latent is
    normalised (MLA post, section 3.5 ``norm_ckv``) and the key part rotated at
    the token's position (section 3.6 Decoupled RoPE, ``denseKR`` + RoPE in
    section 3.7).  Returns (T, dc + dr).
    """
    x = _f64(x)
    a = x @ _f64(w_kva).T
    dc = shape.kv_lora
    c = rms_norm(a[:, :dc], kv_norm_g, shape.rms_eps)
    k_r = rope(a[:, dc:], _f64(pos), shape.rope_base, shape.theta)
    return np.concatenate([c, k_r], axis=1)


def query_heads(x, pos, w: dict, shape: MLAShape):
    """Per-head query parts (q_nope, RoPE(q_rope)), each (T, H, .).

    Without query LoRA: q = W_q x.  With it (MLA post, section 3.1: the query is
    compressed too; section 3.5 ``norm_cq``): q = W_qb RMSNorm(W_qa x).  Each
    head's slice is [q_nope | q_rope] and RoPE is applied per head (section 3.7,
    ``_apply_embeddings``: embedding is done per head).
    """
    x = _f64(x)
    H, dn, dr = shape.n_heads, shape.qk_nope, shape.qk_rope
    if shape.q_lora:
        cq = rms_norm(x @ _f64(w["w_qa"]).T, w["q_norm_g"], shape.rms_eps)
        q = cq @ _f64(w["w_qb"]).T
    else:
        q = x @ _f64(w["w_q"]).T
    q = q.reshape(x.shape[0], H, dn + dr)
    q_n = q[..., :dn]
    q_r = rope(q[..., dn:], _f64(pos)[:, None], shape.rope_base, shape.theta)
    return q_n, q_r


def split_kv_b(w_kvb, shape: MLAShape):
    """Split kv_b_proj (H*(dn+dv), dc) into W_UK (H, dn, dc) and W_UV (H, dv, dc).

    "Deepseek V2 Lite Inference Engine in C", MLA notes: kv_b_proj fuses the K
    and V up-projections and each head's K and V rows are interleaved (head h
    owns rows [h*(dn+dv), (h+1)*(dn+dv)): first dn K rows, then dv V rows).
    """
    H, dn, dv, dc = shape.n_heads, shape.qk_nope, shape.v_head, shape.kv_lora
    wb = _f64(w_kvb).reshape(H, dn + dv, dc)
    return wb[:, :dn, :], wb[:, dn:, :]


def expand_kv(c, w_kvb, shape: MLAShape):
    """Non-absorbed up-projection of every latent row: K_nope (S, H, dn) and V
    (S, H, dv).

    MLA post, section 3.2 Code (``denseUK`` / ``denseUV`` applied to the whole
    cached latent); the C-engine notes' first variant ("use original weights")
    computes the same through kv_b_proj.
    """
    c = _f64(c)
    H, dn, dv = shape.n_heads, shape.qk_nope, shape.v_head
    kv = (c @ _f64(w_kvb).T).reshape(c.shape[0], H, dn + dv)
    return kv[..., :dn], kv[..., dn:]


def _softmax_last(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_attention(q_n, q_r, k_n, k_r, v, q_pos, k_pos, scale: float,
                     return_probs: bool = False):
    """Multi-head attention with decoupled RoPE and a position-offset mask.

    Per head h: K_h = [K_nope_h ; k_rope] (the rope key is shared by all heads,
    MLA post section 3.6 Decoupled RoPE), Q_h = [q_nope_h ; q_rope_h], scores
    s = Q_h . K_h * scale, masked to -inf where the key position is after the
    query position ("Transformer and KV Cache Basics", KV Cache / mask design:
    query positions are offset by the cached length), softmax over keys, then
    the probability-weighted sum of V_h.

    q_n (T,H,dn), q_r (T,H,dr), k_n (S,H,dn), k_r (S,dr), v (S,H,dv).
    Returns o (T, H, dv) [and p (H, T, S) if asked].  Loops over heads to bound
    memory.
    """
    q_n, q_r, k_n, k_r, v = map(_f64, (q_n, q_r, k_n, k_r, v))
    T, H, _ = q_n.shape
    future = np.asarray(q_pos)[:, None] < np.asarray(k_pos)[None, :]
    o = np.empty((T, H, v.shape[-1]), dtype=F64)
    probs = np.empty((H, T, k_n.shape[0]), dtype=F64) if return_probs else None
    for h in range(H):
        qh = np.concatenate([q_n[:, h, :], q_r[:, h, :]], axis=1)
        kh = np.concatenate([k_n[:, h, :], k_r], axis=1)
        s = (qh @ kh.T) * scale
        s[future] = -np.inf
        p = _softmax_last(s)
        o[:, h, :] = p @ v[:, h, :]
        if return_probs:
            probs[h] = p
    return (o, probs) if return_probs else o


def output_projection(o, w_o) -> np.ndarray:
    """y = W_o concat_h(o_h) (MLA post, section 3.2 Code ``denseO``)."""
    o = _f64(o)
    return o.reshape(o.shape[0], -1) @ _f64(w_o).T


def mla_step(x_new, pos_new, rows_prior, w: dict, shape: MLAShape,
             return_probs: bool = False, kv_store=None):
    """One cached MLA step for ONE sequence, non-absorbed.

    The new tokens' latent rows are appended to the cache and the cache is then
    read through the last new position (MLA post, section 3.2 Code: write
    ``cache[:, start_pos:end_pos]`` then read ``1:end_pos``).  Covers decode
    (one new token) and chunked prefill (several), which the KV-cache page
    treats the same way apart from the offset mask.

    x_new (T, D) at positions pos_new (T,); rows_prior (P, R) are the cached
    rows for positions 0..P-1 (P may be 0).  ``kv_store`` (optional) maps the
    rows to what the cache hands back when read (e.g. ``oracle.fp8.fp8_rows``
    for a low-precision cache); it is applied to all rows before attention.
    Returns a dict with the new rows and y (T, D) [and the attention
    probabilities].
    """
    x_new = _f64(x_new)
    pos_new = np.asarray(pos_new)
    rows_new = latent_rows(x_new, pos_new, w["w_kva"], w["kv_norm_g"], shape)
    rows_prior = _f64(rows_prior).reshape(-1, shape.row)
    rows = np.concatenate([rows_prior, rows_new], axis=0)
    if kv_store is not None:
        rows = kv_store(rows)
    dc = shape.kv_lora
    k_n, v = expand_kv(rows[:, :dc], w["w_kvb"], shape)
    q_n, q_r = query_heads(x_new, pos_new, w, shape)
    res = causal_attention(q_n, q_r, k_n, rows[:, dc:], v, pos_new,
                           np.arange(rows.shape[0]), shape.scale, return_probs)
    o, p = res if return_probs else (res, None)
    out = {"rows_new": rows_new, "y": output_projection(o, w["w_o"]), "o": o}
    if return_probs:
        out["p"] = p
    return out


def absorbed_step(x_new, pos_new, rows, w: dict, shape: MLAShape):
    """The same step in weight-absorbed form, fp64, for the identity check and
    for staged intermediates.  ``rows`` are ALL cache rows of the sequence,
    positions 0..S-1, including the new tokens' rows.

    MLA post, section 3.3 Absorption: W_UK is folded into the query side and
    W_UV into the output side (eq. 3.3.3), so scores are taken against the
    latent directly; section 3.6: the rope score is added and the sum scaled
    by 1/sqrt(dn + dr).  Per head:
      q_cat_h = [W_UK_h^T q_nope_h | q_rope_h] * scale         (T, H, R)
      s_h     = q_cat_h . row_t            (all R columns of the cached row)
      o_lat_h = sum_t softmax(s_h)_t c_t                       (T, H, dc)
      o_h     = W_UV_h o_lat_h,   y = W_o concat(o_h)
    """
    rows = _f64(rows)
    pos_new = np.asarray(pos_new)
    dc = shape.kv_lora
    w_uk, w_uv = split_kv_b(w["w_kvb"], shape)
    q_n, q_r = query_heads(x_new, pos_new, w, shape)
    q_abs = np.einsum("thn,hnc->thc", q_n, w_uk)
    q_cat = np.concatenate([q_abs, q_r], axis=-1) * shape.scale
    T, H = q_cat.shape[:2]
    future = pos_new[:, None] < np.arange(rows.shape[0])[None, :]
    o_lat = np.empty((T, H, dc), dtype=F64)
    lse = np.empty((T, H), dtype=F64)
    for h in range(H):
        s = q_cat[:, h, :] @ rows.T
        s[future] = -np.inf
        m = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = np.sum(e, axis=-1, keepdims=True)
        o_lat[:, h, :] = (e / l) @ rows[:, :dc]
        lse[:, h] = (m + np.log(l))[:, 0]
    o = np.einsum("thc,hvc->thv", o_lat, w_uv)
    return {"q_cat": q_cat, "o_lat": o_lat, "lse": lse, "o": o,
            "y": output_projection(o, w["w_o"])}


def decode_batch(x, lengths, rows_per_seq, w: dict, shape: MLAShape):
    """Ragged-batch decode: sequence b has ``lengths[b]`` cached rows (positions
    0..L_b-1, given in ``rows_per_seq[b]``) and one new token x[b] at position
    L_b.  Returns y (B, D) and the new rows (B, R)."""
    x = _f64(x)
    ys, rows_new = [], []
    for b, L in enumerate(lengths):
        r = mla_step(x[b:b + 1], np.array([L]), rows_per_seq[b], w, shape)
        ys.append(r["y"][0])
        rows_new.append(r["rows_new"][0])
    return np.stack(ys), np.stack(rows_new)


def prefill_batch(x, cu_new, prior, rows_prior_per_seq, w: dict, shape: MLAShape,
                  query_subset=None, kv_store=None):
    """Chunked causal prefill: sequence b has ``prior[b]`` cached rows and
    new tokens x[cu_new[b]:cu_new[b+1]] at positions prior[b], prior[b]+1, ...

    ``query_subset`` (optional, per sequence, indices into that sequence's new
    tokens) limits which outputs are computed; all new rows are still appended
    first, so a kept query sees exactly the keys it would in the full run.
    ``kv_store`` (optional) is mla_step's: it maps every key row, cached and
    new, to what the cache hands back when read (the new rows are written
    before they are read), before the expansion.
    Returns a list of (indices, y_rows) per sequence."""
    x = _f64(x)
    out = []
    for b in range(len(prior)):
        xb = x[cu_new[b]:cu_new[b + 1]]
        n = xb.shape[0]
        pos = prior[b] + np.arange(n)
        rows_new = latent_rows(xb, pos, w["w_kva"], w["kv_norm_g"], shape)
        rows = np.concatenate([_f64(rows_prior_per_seq[b]).reshape(-1, shape.row),
                               rows_new], axis=0)
        if kv_store is not None:
            rows = kv_store(rows)
        idx = np.arange(n) if query_subset is None else np.asarray(query_subset[b])
        dc = shape.kv_lora
        k_n, v = expand_kv(rows[:, :dc], w["w_kvb"], shape)
        q_n, q_r = query_heads(xb[idx], pos[idx], w, shape)
        o = causal_attention(q_n, q_r, k_n, rows[:, dc:], v, pos[idx],
                             np.arange(rows.shape[0]), shape.scale)
        out.append((idx, output_projection(o, w["w_o"])))
    return out
