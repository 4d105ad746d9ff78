"""Number-format codecs used by the oracle (TEST INFRASTRUCTURE ONLY).

Written from the public format definitions, not from any library:

* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits;
  the top half of an IEEE-754 binary32.  Encoding rounds to nearest, ties to
  even; overflow goes to infinity; NaN stays NaN.
* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits, no infinities, a single NaN pattern per sign (S.1111.111), largest
  finite magnitude 448, smallest subnormal 2^-9.  Encoding here rounds to
  nearest, ties to even, and saturates finite values to +-448.
* OCP MX FP4: E2M1 elements in blocks of 32 sharing one E8M0 scale (the
  FP4 latent cache of the variants the MLA wiki note's open questions raise).

All arithmetic is float64; every quantisation step below is exact in float64
(scaling by powers of two), so the only rounding is the intended one.

Parity unpinned: the per-row fp8 scale recipe of e4m3_quantize_rows (one
fp32 scale per cache row, max|x| / 448) is a reading; the pages give no fp8
storage recipe.  The codecs themselves are pinned exhaustively.
"""

import numpy as np


def _round_to_grid(a, mant_bits, min_exp):
    """Round non-negative finite float64 values `a` to the nearest value
    with `mant_bits` fractional mantissa bits, exponent >= `min_exp`
    (subnormals below 2^min_exp share the grid spacing 2^(min_exp-mant_bits)).
    Ties go to the even grid point (numpy's round is half-to-even)."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                      # a = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, min_exp)          # exponent of the leading bit
    quantum = np.ldexp(1.0, e - mant_bits)  # spacing of representable values
    return np.round(a / quantum) * quantum


# --------------------------------------------------------------------- bf16
def bf16_decode(bits):
    """uint16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_round(x):
    """float64 -> nearest bfloat16 value (as float64), RNE, overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = _round_to_grid(np.where(np.isfinite(a), a, 0.0), 7, -126)
    max_finite = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > max_finite, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def bf16_encode(x):
    """float64 -> uint16 bfloat16 bit patterns (RNE)."""
    r = bf16_round(x).astype(np.float32)    # exact: bf16 values are binary32 values
    u = r.view(np.uint32) >> np.uint32(16)
    u = np.where(np.isnan(r), np.uint32(0x7FC0), u)
    return u.astype(np.uint16)


# --------------------------------------------------------------- fp8 e4m3fn
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 E4M3 codes -> float64 (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = (m / 8.0) * 2.0 ** -6
    v = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def e4m3_round(x):
    """float64 -> nearest E4M3 value (as float64), RNE, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = _round_to_grid(np.where(np.isfinite(a), a, 0.0), 3, -6)
    r = np.minimum(np.where(np.isinf(a), E4M3_MAX, r), E4M3_MAX)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def e4m3_encode(x):
    """float64 -> uint8 E4M3 codes (RNE, saturating; NaN -> 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(x)
    a = np.abs(np.nan_to_num(r))
    _, e = np.frexp(a)
    e = e - 1
    is_sub = a < 2.0 ** -6
    exp_field = np.where(is_sub, 0, e + 7)
    mant = np.where(is_sub, a / 2.0 ** -9, a / np.ldexp(1.0, e - 3) - 8.0)
    mant = np.where(a == 0, 0, mant)
    exp_field = np.where(a == 0, 0, exp_field)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = code | np.where(np.signbit(r), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def e4m3_quantize_rows(x):
    """Per-row fp8 quantisation of a latent-cache row set.

    One float32 scale per row (token) for all of its elements:
    scale = max|x| / 448 (1 for an all-zero row), code = e4m3(x / scale).
    Returns (codes uint8, scales float32).  The scale is rounded to float32
    first and the division uses that rounded scale, so decode(code)*scale is
    the value a reader of the stored (code, scale) pair reconstructs."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    codes = e4m3_encode(x / scale.astype(np.float64)[..., None])
    return codes, scale


def e4m3_dequantize_rows(codes, scales):
    """(codes, per-row scale) -> float64 rows."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


# ------------------------------------------------------- OCP MX FP4 (E2M1)
# OCP Microscaling (MX) formats v1.0: an MXFP4 block is 32 E2M1 elements
# sharing one E8M0 scale.  E2M1: 1 sign bit, 2 exponent bits (bias 1), 1
# mantissa bit, no infinities or NaN; exponent field 0 is subnormal
# (value m * 2^-1).  E8M0: an 8-bit biased exponent (bias 127), value
# 2^(b - 127), b = 255 is NaN.  The shared scale of a block is
# 2^(floor(log2(max|x|)) - 2) (2 = largest E2M1 exponent); elements are
# x / scale rounded to nearest, ties to even, saturating at +-6.
E2M1_MAX = 6.0
MX_BLOCK = 32


def e2m1_decode(codes):
    """4-bit E2M1 codes (0..15) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    return s * np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))


def e2m1_round(x):
    """float64 -> nearest E2M1 value (as float64), RNE, saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    r = _round_to_grid(np.where(np.isfinite(a), a, 0.0), 1, 0)
    r = np.minimum(np.where(np.isinf(a), E2M1_MAX, r), E2M1_MAX)
    return np.copysign(r, x)


def e2m1_encode(x):
    """float64 -> 4-bit E2M1 codes (RNE, saturating)."""
    r = e2m1_round(x)
    a = np.abs(r)
    _, e = np.frexp(a)
    e = e - 1                                   # exponent of the leading bit
    is_sub = a < 1.0
    exp_field = np.where(is_sub, 0, e + 1)
    mant = np.where(is_sub, a / 0.5, a / np.ldexp(1.0, e - 1) - 2.0)
    code = (exp_field.astype(np.int64) << 1) | np.rint(mant).astype(np.int64)
    return (code | np.where(np.signbit(r), 0x8, 0)).astype(np.uint8)


def e8m0_decode(b):
    """E8M0 scale bytes -> float64 2^(b - 127) (NaN for 255)."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def mx_fp4_quantize_rows(x):
    """Rows [..., d] (d a multiple of 32) -> (E2M1 codes [..., d] uint8,
    E8M0 scale bytes [..., d/32] uint8).  An all-zero block gets scale 1
    (byte 127).  Exponents are clamped to the E8M0 range."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(x.shape[:-1] + (-1, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = f 2^e, f in [0.5, 1)
    shared = np.where(amax > 0, (e - 1) - 2, 0)        # floor(log2(amax)) - emax(E2M1)
    shared = np.clip(shared, -127, 127)
    codes = e2m1_encode(blocks / np.ldexp(1.0, shared)[..., None])
    return codes.reshape(x.shape), (shared + 127).astype(np.uint8)


def mx_fp4_dequantize_rows(codes, scale_bytes):
    """(E2M1 codes [..., d], E8M0 bytes [..., d/32]) -> float64 rows."""
    v = e2m1_decode(codes)
    blocks = v.reshape(v.shape[:-1] + (-1, MX_BLOCK))
    return (blocks * e8m0_decode(scale_bytes)[..., None]).reshape(v.shape)


def unpack_nibbles(packed, n):
    """Bytes holding two 4-bit codes each (element 2i in the low nibble of
    byte i, element 2i+1 in the high one) -> the first n codes, uint8."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (-1,))
    return out[..., :n]
