"""Pins for the numpy e2m3 model (tests/e2m3.py) against the format's
definition (OCP Microscaling Formats specification, e2m3 element type) and
brute force: the value set, nearest-value encoding with ties to the even code,
sign handling, saturation, the block-scale rule and the 6-bit packing."""
import numpy as np

import e2m3


def _all_values():
    return np.array([e2m3.decode(c) for c in range(64)])


def test_value_set():
    mag = e2m3.MAG
    assert mag.shape == (32,) and np.all(np.diff(mag) > 0)
    assert mag[1] == 0.125 and mag[7] == 0.875 and mag[8] == 1.0 and mag[31] == 7.5
    # every normal binade holds 8 evenly spaced values
    for e in range(1, 4):
        seg = mag[8 * e:8 * e + 8]
        np.testing.assert_allclose(np.diff(seg), 2.0 ** (e - 1) / 8)
    # bit layout: sign in bit 5, exponent bits 4-3, mantissa bits 2-0
    assert e2m3.decode(0b011111) == 7.5 and e2m3.decode(0b111111) == -7.5
    assert e2m3.decode(0b001000) == 1.0 and e2m3.decode(0b000001) == 0.125


def test_nearest_value_brute_force():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-7.5, 7.5, 20000), rng.uniform(-1, 1, 5000)])
    vals = _all_values()
    got = e2m3.decode(e2m3.encode(v))
    best = np.abs(v[:, None] - vals[None, :]).min(axis=1)
    np.testing.assert_array_equal(np.abs(v - got), best)


def test_ties_go_to_the_even_code():
    # midpoints between neighbours: the code with mantissa bit 0 clear wins
    for v, code in [(0.0625, 0), (0.1875, 2), (0.9375, 8), (1.0625, 8), (1.1875, 10), (2.125, 16),
                     (3.875, 24), (7.25, 30), (6.75, 30)]:
        assert e2m3.encode(v) == code, (v, e2m3.encode(v), code)
        assert e2m3.encode(-v) == code | 32


def test_saturation_and_zero():
    assert e2m3.encode(7.6) == 31 and e2m3.encode(1e9) == 31 and e2m3.encode(-100.0) == 63
    assert e2m3.decode(e2m3.encode(0.0)) == 0.0 and e2m3.decode(e2m3.encode(0.06)) == 0.0


def test_scale_rule_brute_force():
    rng = np.random.default_rng(4)
    m = np.concatenate([rng.uniform(0, 1, 500) * 2.0 ** rng.integers(-130, 40, 500),
                        [0.0, 7.5, 7.5000005, 3.75, 15.0, 15.000001, 2.0 ** -140]]).astype(np.float32)
    for lo in (-126, -122):
        e = e2m3.scale_exp(m, lo)
        for x, ex in zip(m.astype(np.float64), e):
            want = lo
            while x > 7.5 * 2.0 ** want:
                want += 1
            assert ex == want, (x, lo, ex, want)


def test_pack_layout():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 64, (7, 16))
    b = e2m3.pack16(codes)
    assert b.shape == (7, 12) and b.dtype == np.uint8
    np.testing.assert_array_equal(e2m3.unpack16(b), codes)
    # code i occupies bits 6i .. 6i + 5 of the little-endian field
    one = np.zeros(16, np.int64)
    one[5] = 0b100001
    word = int.from_bytes(bytes(e2m3.pack16(one)), "little")
    assert word == 0b100001 << 30
