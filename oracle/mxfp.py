"""FP8 (E4M3FN, E5M2), FP4 (E2M1), E8M0 and MX group quantization, in float64.

MegaMoE page, "A8W8-FP quantization scenario", stage 1: Q_MX takes groups of
32 consecutive elements, extracts a shared exponent per group (an E8M0 scale
factor) and quantizes the group to FLOAT8_E4M3FN or FLOAT8_E5M2; DQ_MX is the
inverse, done implicitly inside the matmul. The pages do not state the scale
rule or the element rounding; the oracle takes the OCP Microscaling (MX) v1.0
definitions, the standard meaning of a per-group shared exponent stored as E8M0:

* shared exponent  X = 2^(floor(log2(amax)) - emax_elem), emax_elem = 8 (E4M3)
  or 15 (E5M2), the exponent of the element format's largest normal;
  E8M0 byte = exponent + 127, clamped to [0, 254]; an all-zero group gets 0.
* elements  v / X rounded to the nearest value of the element format, ties to
  the even code, magnitudes above the largest finite value clamped to it
  (never NaN or inf for finite input); the sign is kept, so negative values
  that round to zero become -0 (code 0x80).

Scale storage (moe_token_permute 返回值说明, MegaMoE "MXFP quantization
scenario constraints"): [rows, AlignUp(CeilDiv(cols, 32), 2)] bytes, i.e. pairs
of scales; a padding scale (odd group count) is 0x00.

MXFP4 (quantMode 9 of MoeInitRoutingV3 / moe_token_permute): FLOAT4_E2M1 elements
(1 sign, 2 exponent bits with bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3,
4, 6; no inf or NaN), emax_elem = 2, the same E8M0 scale rule and storage. Two
codes share a byte (moe_token_permute: hidden dimension H / 2 in bytes); reading:
element 2j in the low nibble, 2j + 1 in the high nibble (pack_fp4).
"""

from __future__ import annotations

import functools

import numpy as np

GROUP = 32

# name -> (exponent bits, mantissa bits, bias, has_inf)
FORMATS = {
    "e4m3": (4, 3, 7, False),   # FLOAT8_E4M3FN: no inf, only S.1111.111 is NaN
    "e5m2": (5, 2, 15, True),   # FLOAT8_E5M2: IEEE-like inf and NaN
    "e2m1": (2, 1, 1, False),   # FLOAT4_E2M1: every code finite
}
EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}


def code_bits(fmt: str) -> int:
    eb, mb, _, _ = FORMATS[fmt]
    return 1 + eb + mb


@functools.lru_cache(maxsize=None)
def _decode_table(fmt: str) -> np.ndarray:
    eb, mb, bias, has_inf = FORMATS[fmt]
    nbits = code_bits(fmt)
    out = np.empty(1 << nbits, dtype=np.float64)
    for code in range(1 << nbits):
        sign = -1.0 if code >> (nbits - 1) else 1.0
        e = (code >> mb) & ((1 << eb) - 1)
        m = code & ((1 << mb) - 1)
        if e == (1 << eb) - 1 and has_inf:
            val = np.inf if m == 0 else np.nan
        elif e == (1 << eb) - 1 and m == (1 << mb) - 1 and not has_inf and nbits == 8:
            val = np.nan
        elif e == 0:
            val = m * 2.0 ** (1 - bias - mb)          # subnormal
        else:
            val = (1.0 + m / (1 << mb)) * 2.0 ** (e - bias)
        out[code] = sign * val
    out.setflags(write=False)
    return out


def decode_table(fmt: str) -> np.ndarray:
    """float64[2^bits]: the value of every code, from the sign/exponent/mantissa fields."""
    return _decode_table(fmt)


def max_finite(fmt: str) -> float:
    t = decode_table(fmt)
    return float(np.nanmax(t[np.isfinite(t)]))


def e8m0_value(b) -> np.ndarray:
    """E8M0 byte b -> 2^(b-127) (b = 255 is NaN and never produced here)."""
    b = np.asarray(b, dtype=np.int64)
    return np.ldexp(1.0, b - 127)


def scale_cols(cols: int) -> int:
    """AlignUp(CeilDiv(cols, 32), 2)."""
    g = -(-cols // GROUP)
    return g + (g & 1)


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """Exact floor(log2(a)) for positive finite a (frexp gives a = m 2^e, m in [0.5, 1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def round_to_format(y: np.ndarray, fmt: str) -> np.ndarray:
    """Codes of y (already divided by the group scale): nearest value, ties to the
    even code, clamped to +-max finite, sign kept (-0 and negative underflow -> 0x80).
    Done by searching the table of the format's non-negative finite values, which is
    increasing in the code (0x00 .. max code). FP4 codes use 4 bits (sign 0x8)."""
    table = decode_table(fmt)
    top = max_finite(fmt)
    half = len(table) // 2
    pos_codes = np.array([c for c in range(half) if np.isfinite(table[c])], dtype=np.int64)
    pos_vals = table[pos_codes]
    assert np.all(np.diff(pos_vals) > 0)
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), top)
    hi = np.searchsorted(pos_vals, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    d_lo = a - pos_vals[lo]
    d_hi = pos_vals[hi] - a
    c_lo = pos_codes[lo]
    c_hi = pos_codes[hi]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (c_hi % 2 == 0))
    code = np.where(pick_hi, c_hi, c_lo)
    code = np.where(a == pos_vals[hi], c_hi, code)            # exact hits
    neg = np.signbit(y)
    return (code | np.where(neg, half, 0)).astype(np.uint8)


def quantize(v, fmt: str):
    """Q_MX along the last axis.

    v: array [..., C] of finite values (any float dtype; taken exactly as float64).
    Returns (codes uint8 [..., C], scales uint8 [..., AlignUp(CeilDiv(C,32),2)]).
    Rows are independent; large inputs are processed a block of rows at a time.
    """
    v = np.asarray(v)
    cols = v.shape[-1]
    lead = v.shape[:-1]
    flat = v.reshape(-1, cols)
    step = max(1, (1 << 16) // max(cols, 1))
    if flat.shape[0] > step:
        codes = np.empty(flat.shape, dtype=np.uint8)
        scales = np.empty((flat.shape[0], scale_cols(cols)), dtype=np.uint8)
        for lo in range(0, flat.shape[0], step):
            codes[lo:lo + step], scales[lo:lo + step] = _quantize_rows(flat[lo:lo + step], fmt)
        return codes.reshape(lead + (cols,)), scales.reshape(lead + (scale_cols(cols),))
    c, s = _quantize_rows(flat, fmt)
    return c.reshape(lead + (cols,)), s.reshape(lead + (scale_cols(cols),))


def _quantize_rows(v, fmt: str):
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "MX quantization input must be finite"
    cols = v.shape[-1]
    ngroups = -(-cols // GROUP)
    lead = v.shape[:-1]
    padded = np.zeros(lead + (ngroups * GROUP,), dtype=np.float64)
    padded[..., :cols] = v
    g = padded.reshape(lead + (ngroups, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    safe = np.where(amax > 0, amax, 1.0)
    b = _floor_log2(safe) - EMAX[fmt] + 127
    b = np.clip(b, 0, 254)
    b = np.where(amax > 0, b, 0)
    x = e8m0_value(b)
    codes = round_to_format(g / x[..., None], fmt)
    codes = codes.reshape(lead + (ngroups * GROUP,))[..., :cols]
    scales = np.zeros(lead + (scale_cols(cols),), dtype=np.uint8)
    scales[..., :ngroups] = b.astype(np.uint8)
    return np.ascontiguousarray(codes), scales


def pack_fp4(codes) -> np.ndarray:
    """FP4 codes [..., C] (C even) -> bytes [..., C/2]: element 2j low nibble, 2j+1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0 and np.all(c < 16)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize(codes, scales, fmt: str) -> np.ndarray:
    """DQ_MX: value(code) * 2^(scale - 127), scale shared by each 32-group."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    cols = codes.shape[-1]
    vals = decode_table(fmt)[codes]
    grp = np.arange(cols) // GROUP
    return vals * e8m0_value(scales[..., grp])


def bf16_round(v) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest even, one rounding from float64).
    Returns float64 values that are exactly representable in bf16."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    e = _floor_log2(np.abs(v[nz]))
    e = np.maximum(e, -126)                   # bf16 subnormals share the 2^-133 quantum
    q = np.ldexp(1.0, e - 7)                  # 8 significant bits
    out[nz] = np.rint(v[nz] / q) * q          # np.rint rounds half to even
    out[~nz] = v[~nz]
    return out


def bf16_bits(v) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float64 values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def fp32_round(v) -> np.ndarray:
    """float64 -> nearest fp32 (IEEE RNE), returned as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
