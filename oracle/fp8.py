"""FP8 e4m3fn and e8m0 codecs, written out from the OCP 8-bit float formats.

e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, S.1111.111 is NaN; largest finite 448 = 2^8 * 1.75.
Normal: (-1)^s * 2^(e-7) * (1 + m/8); subnormal (e = 0): (-1)^s * 2^-6 * m/8.
e8m0: an unsigned biased exponent, value 2^(c-127), code 255 is NaN.

These formats are the block-FP8 weights of the DSV2-236B-MegaKernel README
("Results": per-128 block-scaled FP8; "Layout": E4M3 with UE8M0 scales) and
the MXFP8 routed experts of Mixture-of-Kittens (Table 2 caption).
Pinned by tests against torch.float8_e4m3fn on all 256 codes and on
round-to-nearest-even midpoints.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    v = s * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(values):
    """float64 (finite) -> uint8 codes: round to nearest, ties to even, saturating at +-448."""
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: a < 2^-6, steps of 2^-9
    sub = a < 2.0 ** -6
    msub = np.rint(a * 2.0 ** 9).astype(np.int64)          # 0..8; 8 is the smallest normal
    code = np.where(sub, msub, code)
    # normal range: a = 2^E * f, f in [1, 2)
    f, ex = np.frexp(np.where(sub, 1.0, a))                # a = f' * 2^ex, f' in [0.5, 1)
    E = ex - 1
    with np.errstate(invalid="ignore"):                    # NaN inputs give an arbitrary code
        mant = np.rint((f * 2.0 - 1.0) * 8.0).astype(np.int64)  # 0..8, ties to even
    E = np.where(mant == 8, E + 1, E)
    mant = np.where(mant == 8, 0, mant)
    ncode = ((E + 7) << 3) | mant
    ncode = np.minimum(ncode, 0x7E)                        # saturate (448 is 0x7E)
    code = np.where(sub, code, ncode)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def e8m0_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))
