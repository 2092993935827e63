"""Exact decoders and round-to-nearest-even encoders for the formats on the path.

Test infrastructure (see the package docstring); never used by the product path.

Formats (radiance_mxfp4.py page, ``_exact_ref`` and ``_traced_quant``;
radiance_kernels.py page, the e4m3fn weight guard in ``install_load_hook``):
  e4m3fn  OCP FP8: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity,
          0x7F/0xFF are NaN, largest finite 448.
  e2m1    OCP FP4: 1 sign, 2 exponent (bias 1), 1 mantissa bit; the page's
          lookup table is [0, .5, 1, 1.5, 2, 3, 4, 6] with bit 3 the sign.
  e8m0    MX block scale: 2**(e - 127); 255 is NaN (OCP MX; the pages never
          produce it).
  bf16    the upper 16 bits of an IEEE binary32.
"""
import numpy as np


# ----------------------------------------------------------------- decoders
def decode_e4m3(codes):
    """e4m3fn code -> exact value (fp64).  Subnormals: m * 2**-9."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_e2m1(nibbles):
    """e2m1 code (low 4 bits) -> exact value (fp64)."""
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 15
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (2 + m) * np.exp2(e - 2.0))
    return np.where(s == 1, -mag, mag)


def decode_e8m0(exps):
    """e8m0 exponent byte -> 2**(e-127) (fp64); 255 -> NaN."""
    e = np.asarray(exps, dtype=np.uint8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def decode_bf16(bits):
    """bf16 bit pattern (uint16) -> exact value (fp64)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def unpack_fp4(packed):
    """[..., K/2] uint8 -> [..., K] e2m1 codes.  Element 2j is the low nibble
    of byte j, element 2j+1 the high nibble (radiance_mxfp4.py page,
    ``_exact_ref``: codes are (b & 0xF, b >> 4) interleaved)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------- encoders
def _floor_log2(a):
    """floor(log2 a) for finite a > 0, exact (frexp: a = f * 2**x, f in [.5,1))."""
    _, x = np.frexp(a)
    return x.astype(np.int64) - 1


def round_to_fp32(x):
    """One IEEE round-to-nearest-even from fp64 to binary32 (library cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16(x):
    """fp64 -> bf16 bit pattern, ONE round-to-nearest-even of the fp64 value
    (no double rounding through fp32).  Subnormal bf16 has quantum 2**-133;
    magnitudes that round to 2**128 or beyond become infinity; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    safe = np.where((a > 0) & np.isfinite(a), a, 1.0)
    e = np.maximum(_floor_log2(safe), -126)          # subnormals share 2**-126's quantum
    quantum = np.exp2(e - 7.0)
    r = np.rint(safe / quantum) * quantum            # np.rint: ties to even
    r = np.where(a == 0, 0.0, r)
    r = np.where(np.isinf(a) | (r >= 2.0 ** 128), np.inf, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def round_to_e4m3(x):
    """fp64 value with |x| <= 448 -> e4m3fn code, round to nearest, ties to even.
    Below 2**-6 the quantum is 2**-9 (subnormals); a carry into the next binade
    is handled by re-deriving the exponent from the rounded value.  Negative
    values that round to zero give 0x80."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~(a <= 448.0)):
        raise ValueError("round_to_e4m3 needs |x| <= 448 (clamp first); NaN is not encoded")
    safe = np.where(a > 0, a, 1.0)
    e = np.maximum(_floor_log2(safe), -6)
    quantum = np.exp2(e - 3.0)
    r = np.where(a > 0, np.rint(safe / quantum) * quantum, 0.0)
    sub = r < 2.0 ** -6
    code_sub = np.rint(r * 2.0 ** 9).astype(np.int64)                 # m, exponent field 0
    rs = np.where(sub, 1.0, r)
    e2 = _floor_log2(rs)
    m2 = np.rint(rs * np.exp2(3.0 - e2) - 8).astype(np.int64)
    code_norm = ((e2 + 7) << 3) | m2
    code = np.where(sub, code_sub, code_norm)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------- lattice helpers
def e4m3_step_index(codes):
    """Position of an e4m3 code on the value-ordered lattice, with +0 == -0.
    Codes 0x00..0x7E increase with value, so the index is the code for
    positives and minus the magnitude code for negatives.  NaN codes map far
    away so that any comparison with them fails."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    idx = np.where(c >= 0x80, -mag, mag)
    return np.where(mag == 0x7F, 10 ** 6, idx)


def bf16_ulp(x):
    """Size of one bf16 ulp at |x|: 2**(floor(log2|x|) - 7), 2**-133 below 2**-126."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    safe = np.where(a > 0, a, 1.0)
    e = np.maximum(_floor_log2(safe), -126)
    return np.where(a >= 2.0 ** -126, np.exp2(e - 7.0), 2.0 ** -133)
