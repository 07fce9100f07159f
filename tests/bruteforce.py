"""Pure-Python brute-force MLA, used only to pin the fp64 oracle on tiny inputs.

Written independently of ``oracle/`` from the pages' definitions, in a
different shape of code: Python floats and lists, explicit loops, complex
numbers for RoPE, materialised per-head keys and values, and the per-query
attention sum of "Transformer and KV Cache Basics" (KV Cache, conceptually:
scores over k_1..k_n, softmax, sum of score_i * v_i).
"""

import cmath
import math


def _matvec(W, x):
    return [sum(W[i][j] * x[j] for j in range(len(x))) for i in range(len(W))]


def _rmsnorm(v, g, eps):
    r = math.sqrt(sum(t * t for t in v) / len(v) + eps)
    return [v[i] / r * g[i] for i in range(len(v))]


def _rope(v, pos, base):
    # MLA post section 3.7: adjacent pairs as complex numbers times
    # (cos + i sin) of pos * theta_i, theta_i = 1 / base^(2i/d)
    d = len(v)
    out = []
    for i in range(d // 2):
        theta = 1.0 / (base ** ((2 * i) / d))
        z = complex(v[2 * i], v[2 * i + 1]) * cmath.exp(1j * pos * theta)
        out += [z.real, z.imag]
    return out


def mla_brute(xs, positions_new, n_prior, W, dims, eps=1e-6, base=10000.0):
    """Outputs of the new tokens of ONE sequence.

    xs: list of all token hidden vectors (prior tokens first, then the new
    ones); the prior tokens are at positions 0..n_prior-1 and the new ones at
    ``positions_new``.  W: dict of nested lists (row-major (out, in)).
    """
    H, dn, dr, dv, dc = (dims["n_heads"], dims["qk_nope"], dims["qk_rope"],
                         dims["v_head"], dims["kv_lora"])
    dq = dims.get("q_lora", 0)
    positions = list(range(n_prior)) + list(positions_new)
    # latent rows of every token (written to the cache first)
    cache = []
    for x, p in zip(xs, positions):
        a = _matvec(W["w_kva"], x)
        c = _rmsnorm(a[:dc], W["kv_norm_g"], eps)
        kr = _rope(a[dc:], p, base) if dr else []
        cache.append((c, kr))
    # materialised per-head keys / values: kv_b rows per head are [K (dn); V (dv)]
    K = [[None] * len(cache) for _ in range(H)]
    V = [[None] * len(cache) for _ in range(H)]
    for t, (c, kr) in enumerate(cache):
        for h in range(H):
            base_row = h * (dn + dv)
            kn = _matvec(W["w_kvb"][base_row:base_row + dn], c)
            vv = _matvec(W["w_kvb"][base_row + dn:base_row + dn + dv], c)
            K[h][t] = kn + kr
            V[h][t] = vv
    ys = []
    for k, x in enumerate(xs[n_prior:]):
        p = positions_new[k]
        if dq:
            q = _matvec(W["w_qb"], _rmsnorm(_matvec(W["w_qa"], x), W["q_norm_g"], eps))
        else:
            q = _matvec(W["w_q"], x)
        o = []
        for h in range(H):
            qh = q[h * (dn + dr):(h + 1) * (dn + dr)]
            qh = qh[:dn] + (_rope(qh[dn:], p, base) if dr else [])
            scale = 1.0 / math.sqrt(dn + dr)
            visible = [t for t in range(len(cache)) if positions[t] <= p]
            s = [sum(qh[i] * K[h][t][i] for i in range(dn + dr)) * scale for t in visible]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            oh = [0.0] * dv
            for w_, t in zip(e, visible):
                for i in range(dv):
                    oh[i] += (w_ / z) * V[h][t][i]
            o += oh
        ys.append(_matvec(W["w_o"], o))
    return ys
