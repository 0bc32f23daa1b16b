"""The p-record check of tests/test_gpu_sampler.py::test_p_image_records, on
the CPU: records built by the numpy model pass it (also with the weights
perturbed by the size of the device's exp2 error), and the plausible
mistakes fail it: every code encoded under a scale one too large, the scale
byte one too large for the codes, the two code sets swapped, the residual
scaled by 2^10 instead of 2^11, a nonzero padding byte."""
import numpy as np
import pytest

import e2m3
import p_records as PR


def _weights(seed=0):
    rng = np.random.default_rng(seed)
    p = np.exp2(rng.uniform(-30, 0, (64, 40, 16))) * np.exp2(14 - rng.integers(0, 20, (64, 40, 16)))
    return p.astype(np.float32)


def test_model_records_pass():
    pref = _weights()
    PR.check_records(PR.encode_records(pref), pref)
    # the device's P' differs from the reference by ~2^-20 relative
    jitter = (pref * (1 + np.float32(2.0 ** -21) * np.sign(np.random.default_rng(1).standard_normal(pref.shape)))
              ).astype(np.float32)
    PR.check_records(PR.encode_records(jitter), pref)


def _mutate(rec, pref, kind):
    rec = rec.copy()
    if kind == "scale_up":
        es = rec[..., 56].astype(np.int64) - 116 + 1
        sc = np.exp2(es.astype(np.float64))[..., None]
        p16 = rec[..., :32].copy().view(np.float16).astype(np.float64).reshape(pref.shape)
        r16 = ((pref - p16.astype(np.float32)) * np.float32(2048.0)).astype(np.float16).astype(np.float64)
        rec[..., 32:44] = e2m3.pack16(e2m3.encode(p16 / sc))
        rec[..., 44:56] = e2m3.pack16(e2m3.encode(r16 / sc))
        rec[..., 56] = (116 + es).astype(np.uint8)
    elif kind == "scale_byte":
        rec[..., 56] += 1
    elif kind == "swap_sets":
        a = rec[..., 32:44].copy()
        rec[..., 32:44] = rec[..., 44:56]
        rec[..., 44:56] = a
    elif kind == "residual_2_10":
        p16 = rec[..., :32].copy().view(np.float16).astype(np.float32).reshape(pref.shape)
        es = rec[..., 56].astype(np.int64) - 116
        sc = np.exp2(es.astype(np.float64))[..., None]
        r16 = ((pref - p16) * np.float32(1024.0)).astype(np.float16).astype(np.float64)
        rec[..., 44:56] = e2m3.pack16(e2m3.encode(r16 / sc))
    elif kind == "padding":
        rec[3, 5, 60] = 1
    return rec


@pytest.mark.parametrize("kind", ["scale_up", "scale_byte", "swap_sets", "residual_2_10", "padding"])
def test_planted_mistakes_fail(kind):
    pref = _weights(2)
    bad = _mutate(PR.encode_records(pref), pref, kind)
    with pytest.raises(AssertionError):
        PR.check_records(bad, pref)
