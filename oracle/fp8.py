"""FP8 formats for the oracle: E4M3 (OCP "FN" variant) and E8M0, written from
their bit-field definitions, plus the quantizers that write a KV cache.

Test infrastructure only (see the package docstring).

Sources.  The method page ("fp8 paged attention for MoE serving") stores K/V as
E4M3 codes with fp32 scales, per (token, head) or per sub-row group, and its
reference dequantizes as ``code value x scale`` (section "Smallest correct
example": ``dequant_kv_fp8_ref(q, s)``).  The MXFP8 page ("Attention MXFP8 TKG
Kernel API Reference") adds E8M0 power-of-two scales shared by 32 elements.
The pages do not spell out the encodings; the readings taken here are:

* E4M3 is the OCP FN variant: bias 7, no infinities, S.1111.111 is NaN, the
  largest finite magnitude is 448.
* E8M0 is the OCP MX scale: value 2**(u-127), u = 255 is NaN.
* Encoding rounds to the nearest finite E4M3 value, ties to the even mantissa
  (= even code), saturating at +-448, keeping the sign (so -0 and negative
  values that round to zero give 0x80).
* fp32 block scale: s = fp32(amax / 448), and s = 1 when amax = 0.
* E8M0 block scale: the smallest power of two 2**k with amax <= 448 * 2**k,
  stored as u = clamp(k + 127, 0, 254); u = 127 when amax = 0.
* The value to encode is y = fp32(x / s), the correctly rounded fp32 quotient
  (computed here in float64 and rounded once to fp32: for a quotient of two
  fp32 numbers that double rounding equals the single correct rounding).
"""
import math

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code: sign bit 7, exponent bits 6..3, mantissa 2..0."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = m * 2.0 ** -9            # subnormal: (m / 8) * 2**(1 - 7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale byte: 2**(code - 127); 255 is NaN."""
    return math.nan if code == 255 else 2.0 ** (code - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
# The 127 non-negative finite codes 0x00..0x7E, strictly increasing in value.
_POS = E4M3_TABLE[:127]


def to_fp32(x):
    """Round float64 values to the nearest fp32 (ties to even), back as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def encode_e4m3(y) -> np.ndarray:
    """Nearest finite E4M3 code to each value of ``y`` (ties to the even code),
    saturating at +-448.  ``y`` must hold no NaN."""
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("encode_e4m3: NaN input")
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")       # _POS[hi-1] < a <= _POS[hi]
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)
    return code


def fp32_scale_from_amax(amax):
    """fp32 block scale fp32(amax / 448); 1.0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    s = to_fp32(amax / E4M3_MAX)
    return np.where(amax == 0.0, 1.0, s)


def e8m0_code_from_amax(amax) -> np.ndarray:
    """E8M0 code of the smallest power of two 2**k with amax <= 448 * 2**k.

    With amax = f * 2**e (f in [0.5, 1)), 448 * 2**(e-9) = 0.875 * 2**e, and
    448 * 2**(e-10) < 2**(e-1) <= amax; so k = e - 9 when f <= 0.875, else e - 8.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(amax)
    k = np.where(f <= 0.875, e - 9, e - 8)
    code = np.clip(k + 127, 0, 254)
    return np.where(amax == 0.0, 127, code).astype(np.uint8)


def quantize_fp32_block(x):
    """One fp32 scale for the whole of ``x``: returns (codes, scale)."""
    x = np.asarray(x, dtype=np.float64)
    s = float(fp32_scale_from_amax(np.abs(x).max() if x.size else 0.0))
    return encode_e4m3(to_fp32(x / s)), s


def quantize_e8m0_g32(x):
    """E8M0 scale per 32 consecutive elements of the last axis.

    Returns (codes with the shape of x, scale codes of shape [..., D // 32])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 32:
        raise ValueError("last axis must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (d // 32, 32))
    u = e8m0_code_from_amax(np.abs(g).max(axis=-1))
    scale = E8M0_TABLE[u][..., None]
    codes = encode_e4m3(to_fp32(g / scale)).reshape(x.shape)
    return codes, u


def dequant(codes, scale):
    """Exact float64 value code x scale (4 x 24 significant bits fit in 53)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)


def dequant_fp32(codes, scale):
    """The fp32 dequantized value: the exact product rounded once to fp32."""
    return to_fp32(dequant(codes, scale))
