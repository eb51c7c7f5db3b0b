"""FP8 (float8 e4m3, the "fn" variant) attention forward: plain fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "nanochat Admin & Developer Guide", section 5 "Precision: Explicit
dtype & FP8": forward operands are float8 e4m3 ("fn": no infinities) with
tensorwise dynamic scaling, i.e. one scale per tensor taken from its
absolute maximum; and section 6 "Attention: FA3 with SDPA Fallback": the
attention kernel accepts fp8 as well as bf16 operands. The attention of fp8
operands is defined here as the attention of their dequantized values,
x = value(code) * descale, one descale per tensor, computed in fp64 by
``attn_fwd``. How a kernel rounds its intermediates (the probabilities fed
to an fp8 product, for instance) is not part of the definition; the tests
bound that rounding separately.

The e4m3 format (8 bits): sign in bit 7; a 4-bit exponent field E (bits
6..3, bias 7); a 3-bit mantissa M (bits 2..0). E = 0 encodes the subnormals
(M / 8) * 2^-6; E = 15 with M = 7 encodes NaN; every other code is
(1 + M / 8) * 2^(E - 7). The largest finite magnitude is 448 (E = 15,
M = 6), the smallest subnormal 2^-9.
"""

import numpy as np

from .attention import attn_fwd

E4M3_MAX = 448.0


def e4m3_value(code):
    """The value of one e4m3 code (an int 0..255); NaN for the NaN codes."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the non-negative finite values in increasing order, with their codes
_POS_CODES = np.array([c for c in range(128) if not np.isnan(_TABLE[c])], dtype=np.int64)
_POS_VALUES = _TABLE[_POS_CODES]


def e4m3_decode(codes):
    """uint8 codes (any shape) -> their fp64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_encode(x):
    """fp64 values -> uint8 codes: the nearest e4m3 value, ties to the code
    with an even mantissa, magnitudes beyond 448 saturated to 448; NaN maps
    to the NaN code 0x7F. The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def tensorwise_descale(x):
    """The tensorwise dynamic scale: amax / 448 (1 for an all-zero tensor),
    so that x / descale spans the whole e4m3 range."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else 0.0
    return amax / E4M3_MAX if amax > 0 else 1.0


def quantize_tensorwise(x):
    """x -> (codes, descale): codes = e4m3_encode(x / descale)."""
    s = tensorwise_descale(x)
    return e4m3_encode(np.asarray(x, dtype=np.float64) / s), s


def attn_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, window, scale):
    """Attention forward of e4m3 codes q8 [B,T,H,D], k8/v8 [B,T,Hkv,D] with
    one descale per tensor: (out, lse) of the dequantized operands."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    v = e4m3_decode(v8) * float(v_descale)
    return attn_fwd(q, k, v, window, scale)
