"""Pins for the oracle's FP8 (OCP E4M3) decoding and FP8 attention (CPU only)."""
import numpy as np
import torch

from oracle import fp8 as F
from oracle.attention import canvas_attention


def test_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_closed_form_codes():
    v = F.e4m3_to_float(np.array([0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x08, 0x00, 0x80, 0x3C, 0x07], np.uint8))
    assert list(v[:6]) == [1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -6]
    assert v[6] == 0.0 and v[7] == 0.0 and np.signbit(v[7])
    assert v[8] == 1.5 and v[9] == 7 * 2.0 ** -9


def test_grid_is_three_mantissa_bits_in_range():
    v = F.e4m3_to_float(np.arange(256, dtype=np.uint8))
    v = v[np.isfinite(v)]
    pos = np.unique(np.abs(v))
    want = {0.0}
    for e in range(-6, 9):                       # normals 2^-6 .. 2^8 * 1.75
        for m in range(8):
            x = (1 + m / 8) * 2.0 ** e
            if x <= 448:
                want.add(x)
    want |= {m / 8 * 2.0 ** -6 for m in range(1, 8)}
    assert set(pos.tolist()) == want


def codes(rng, shape, std=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_attention_is_the_plain_definition_on_decoded_values():
    rng = np.random.default_rng(0)
    q, kp, vp, kc, vc = (codes(rng, s) for s in [(6, 4, 64), (9, 2, 64), (9, 2, 64), (6, 2, 64), (6, 2, 64)])
    o = F.canvas_attention_fp8(q, kp, vp, kc, vc, q_scale=0.5, k_scale=2.0, v_scale=3.0)
    d = lambda x, s: F.e4m3_to_float(x) * s
    ref = canvas_attention(d(q, 0.5), d(kp, 2.0), d(vp, 3.0), d(kc, 2.0), d(vc, 3.0))
    np.testing.assert_allclose(o, ref, rtol=1e-14, atol=1e-14)


def test_scale_placement():
    rng = np.random.default_rng(1)
    q, kp, vp, kc, vc = (codes(rng, s) for s in [(5, 2, 64), (7, 1, 64), (7, 1, 64), (5, 1, 64), (5, 1, 64)])
    a = F.canvas_attention_fp8(q, kp, vp, kc, vc, q_scale=2.0, k_scale=0.25)
    b = F.canvas_attention_fp8(q, kp, vp, kc, vc, q_scale=0.5, k_scale=1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    c = F.canvas_attention_fp8(q, kp, vp, kc, vc, q_scale=2.0, k_scale=0.25, v_scale=4.0)
    np.testing.assert_allclose(c, 4.0 * a, rtol=1e-13)
    # zero keys: every weight equal, O is the mean of the decoded values
    z = np.zeros_like(kp), np.zeros_like(kc)
    m = F.canvas_attention_fp8(q, z[0], vp, z[1], vc)
    mean = np.concatenate([F.e4m3_to_float(vp), F.e4m3_to_float(vc)]).mean(axis=0)
    np.testing.assert_allclose(m[:, 0], np.broadcast_to(mean[0], (5, 64)), rtol=1e-13, atol=1e-15)
