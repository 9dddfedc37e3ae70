"""Number formats for the oracle, written from their definitions (fp64 numpy).

bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits -- the top half of an
IEEE binary32.  Rounding to bf16 is round-to-nearest, ties to even, with
values past the largest finite bf16 going to infinity.

OCP E4M3FN ("OCP 8-bit Floating Point Specification", E4M3 encoding):
1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity; the largest
finite magnitude is S.1111.110 = 448.

The pages' own low-bit formats are never defined, so the fp8 workload uses
this standard format (gfx950 converts it natively).  Encoding here is
round-to-nearest-even and saturates magnitudes >= 448 to 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the bf16 grid (RNE), returned as fp64.

    For |x| with leading-bit exponent ex (x = m * 2^ex, 1 <= m < 2) the bf16
    spacing is 2^(max(ex, -126) - 7); below 2^-126 the spacing stays 2^-133
    (subnormals).  Results at or above 2^128 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if np.any(fin):
        v = x[fin]
        _, e2 = np.frexp(np.abs(v))  # |v| = fr * 2^e2, 0.5 <= fr < 1
        ex = np.maximum(e2 - 1, -126)
        ulp = np.ldexp(1.0, ex - 7)
        r = np.rint(v / ulp) * ulp  # v / ulp is exact: ulp is a power of two
        r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
        out[fin] = r
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> fp64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = sign * mag
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return val


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> OCP E4M3FN codes, round-to-nearest-even, saturating.

    |v| >= 448 gives +-448 (code 0x7E / 0xFE); NaN gives 0x7F; the sign of
    zero is kept (a negative value that rounds to zero gives 0x80).
    """
    with np.errstate(invalid="ignore"):
        v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    codes = np.zeros(v.shape, dtype=np.int64)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, a)
    sat = a >= E4M3_MAX
    # quantum of the binade that holds a (subnormal quantum 2^-9 below 2^-6)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))
    ex = np.maximum(e2 - 1, -6)
    q = np.ldexp(1.0, ex - 3)
    n = np.rint(a / q)  # exact scaling by a power of two, then RNE
    r = n * q  # rounded magnitude, may have moved up one binade
    # encode r (for r < 448 only; saturated lanes are overwritten below)
    _, re2 = np.frexp(np.where(r > 0, r, 1.0))
    rex = re2 - 1
    normal = (r >= 2.0 ** -6)
    e_field = np.where(normal, rex + 7, 0)
    m_field = np.where(normal, np.rint((r / np.ldexp(1.0, rex) - 1.0) * 8.0), np.rint(r / 2.0 ** -9))
    m_field = np.where((r == 0) | sat, 0, m_field)
    e_field = np.where((r == 0) | sat, 0, e_field)
    codes = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    codes = np.where(sat, 0x7E, codes)
    codes = codes | np.where(sign, 0x80, 0)
    codes = np.where(nan, 0x7F, codes)
    return codes.astype(np.uint8)


def quant_row_fp8(row_f32: np.ndarray):
    """Quantise one activation row to E4M3 with one fp32 scale.

    s = fp32(max|v|) / 448 by IEEE fp32 division; q = e4m3(fp32(v) / s) by
    IEEE fp32 division (no reciprocal).  An all-zero row gives s = 1, q = 0.
    Returns (codes uint8, scale float32).
    """
    v = np.asarray(row_f32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    if amax == 0:
        return np.zeros(v.shape, dtype=np.uint8), np.float32(1.0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    scaled = (v / s).astype(np.float32)
    return e4m3_encode(scaled), s


def quant_rows_fp8(rows_f32: np.ndarray):
    """Row-wise ``quant_row_fp8`` over a 2-D array."""
    rows = np.asarray(rows_f32, dtype=np.float32)
    q = np.empty(rows.shape, dtype=np.uint8)
    s = np.empty(rows.shape[0], dtype=np.float32)
    for i in range(rows.shape[0]):
        q[i], s[i] = quant_row_fp8(rows[i])
    return q, s


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))
