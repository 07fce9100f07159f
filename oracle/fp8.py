"""FP8 latent-cache storage for the oracle: OCP E4M3 codes with one scale per row.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "Multi-Head Latent Attention" post lists low-precision storage among
DeepSeek's implementation ideas (introduction) and sizes a cache element at
1 byte for FP8 (section 3.1 C cache); it gives no quantisation formula.
Reading: the latent part c (d_c values) of each
cached row is stored as OCP FP8 E4M3 codes with one fp32 scale per row,
    s = max_i |c_i| / 448   (s = 1 for an all-zero row),
    code_i = E4M3(c_i / s)  (round to nearest, ties to even, saturating at +-448),
and read back as c_i ~= s * value(code_i); the shared RoPE key k_rope stays in
bf16 (it is rotated per position and only d_r wide).  E4M3 is the 8-bit float
with 1 sign, 4 exponent (bias 7) and 3 mantissa bits; exponent field 0 holds
the subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN; there are no
infinities; the largest finite magnitude is 448 = 1.75 * 2^8.

Everything here follows that definition directly: decoding is the closed
form, encoding rounds |x| on the grid of the binade it falls in.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_SUB_STEP = 2.0 ** -9        # spacing of the subnormals
_MIN_NORMAL = 2.0 ** -6


def e4m3_decode(code) -> np.ndarray:
    """float64 value of each E4M3 code (uint8); NaN for 0x7F / 0xFF."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, m * _SUB_STEP, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code (uint8) nearest to each finite x, ties to even mantissa,
    |x| beyond 448 clamped to 448.  The sign bit follows x (so -0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # grid spacing of the binade holding a: 2^(E - 3) for a >= 2^-6, else 2^-9
    E = np.floor(np.log2(np.maximum(a, _MIN_NORMAL)))
    step = np.exp2(E - 3.0)
    q = np.round(a / step) * step           # np.round: ties to even
    q = np.minimum(q, E4M3_MAX)
    # code of the (representable) magnitude q
    Eq = np.floor(np.log2(np.maximum(q, _MIN_NORMAL)))
    is_norm = q >= _MIN_NORMAL
    mant_n = np.round((q / np.exp2(Eq) - 1.0) * 8.0)
    code_n = ((Eq + 7.0) * 8.0 + mant_n)
    code_s = np.round(q / _SUB_STEP)
    code = np.where(is_norm, code_n, code_s).astype(np.int64)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_latent(c, f32: bool = False):
    """Row scales and E4M3 codes of latent rows c (T, d_c).

    f32=False: the definition in float64.  f32=True: the same steps in float32
    arithmetic (scale = fp32(max|c|) / 448, q = c / scale, both correctly
    rounded fp32 operations) -- how a GPU kernel computing in fp32 decides
    the codes, for bit-exact comparison on identical fp32 inputs."""
    if f32:
        c = np.asarray(c, dtype=np.float32)
        amax = np.max(np.abs(c), axis=1)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (c / s[:, None]).astype(np.float32)
        return s, e4m3_encode(q.astype(np.float64))
    c = np.asarray(c, dtype=np.float64)
    amax = np.max(np.abs(c), axis=1)
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return s, e4m3_encode(c / s[:, None])


def dequantize_latent(s, codes) -> np.ndarray:
    """c ~= s * value(code), float64 (T, d_c)."""
    return np.asarray(s, dtype=np.float64)[:, None] * e4m3_decode(codes)


def fp8_rows(rows, d_c: int) -> np.ndarray:
    """What an FP8 cache hands back for latent rows [c | k_rope] (T, d_c + d_r):
    the latent part quantised and read back, the rope part unchanged (the
    library stores it in bf16, whose rounding the tolerance covers as in the
    bf16 cache)."""
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return rows.copy()
    s, q = quantize_latent(rows[:, :d_c])
    return np.concatenate([dequantize_latent(s, q), rows[:, d_c:]], axis=1)
