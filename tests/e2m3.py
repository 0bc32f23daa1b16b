"""The e2m3 element format of the OCP Microscaling (MX) specification, in
numpy, from its definition: six bits (sign, two exponent bits of bias 1, three
mantissa bits), no infinities and no NaN.  Exponent field 0 holds the
subnormals m/8; field e >= 1 holds (1 + m/8)·2^(e - 1), up to 7.5.

The packed contraction stores its correction terms in this format under
power-of-two block scales; the tests model those roundings with these
functions, which test_e2m3.py pins against the definition.
"""
import numpy as np

# magnitude of code 0..31 (bit 5 is the sign)
MAG = np.array([m / 8.0 for m in range(8)] +
               [(1.0 + m / 8.0) * 2.0 ** (e - 1) for e in range(1, 4) for m in range(8)])
MAX = 7.5


def encode(v):
    """Nearest e2m3 code of each value (ties to the even code), sign in bit 5;
    magnitudes above 7.5 saturate to 7.5."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(MAG, a), 1, 31)      # MAG[hi - 1] < a <= MAG[hi] inside the range
    lo = hi - 1
    d_lo, d_hi = a - MAG[lo], MAG[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= MAX, 31, code)
    return (code | ((v < 0) << 5)).astype(np.int64)


def decode(c):
    c = np.asarray(c, np.int64)
    return np.where(c & 32, -1.0, 1.0) * MAG[c & 31]


def scale_exp(m, lo):
    """The smallest integer e >= lo with m <= 7.5·2^e (m >= 0, float32)."""
    m = np.asarray(m, np.float32).astype(np.float64)
    e = np.full(m.shape, lo, np.int64)
    pos = m > 0
    fr, ex = np.frexp(m[pos])                          # m = fr·2^ex, fr in [0.5, 1)
    e[pos] = np.maximum(ex - 3 + (fr > 0.9375), lo)    # 7.5·2^e = 0.9375·2^(e + 3)
    return e


def pack16(codes):
    """[..., 16] codes -> [..., 12] bytes: code i at bits 6i..6i+5 of the
    little-endian 96-bit field."""
    codes = np.asarray(codes, np.int64)
    bits = (codes[..., :, None] >> np.arange(6)) & 1                  # [..., 16, 6]
    bits = bits.reshape(*codes.shape[:-1], 96)
    return (bits.reshape(*codes.shape[:-1], 12, 8) << np.arange(8)).sum(-1).astype(np.uint8)


def unpack16(b):
    b = np.asarray(b, np.int64)
    bits = ((b[..., :, None] >> np.arange(8)) & 1).reshape(*b.shape[:-1], 96)
    return (bits.reshape(*b.shape[:-1], 16, 6) << np.arange(6)).sum(-1)
