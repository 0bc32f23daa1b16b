"""The sampler's p records (fp16 + fp6 split of one row's 16 weights of a
k-block) in numpy: a model that builds them from the shifted weights P', and
the check the GPU test applies to the records the statistics pass writes.

Record layout (64 bytes): fp16 P'16 of ids 0-15; 32 e2m3 codes, six bytes per
eight codes, code i at bits 6i of the 24 bytes (P'16 of ids 0-15, then
r = fp16((P' - P'16) 2^11) of ids 0-15) divided by 2^es, es the smallest
exponent (at least -116) that brings all 32 fp16 values to 7.5 or below; the
byte 116 + es; seven zero bytes.
"""
import numpy as np

import e2m3


def encode_records(pref):
    """[..., 16] float32 P' -> [..., 64] uint8 records."""
    pref = np.asarray(pref, np.float32)
    p16 = pref.astype(np.float16)
    r16 = ((pref - p16.astype(np.float32)) * np.float32(2048.0)).astype(np.float16)
    mx = np.maximum(p16.astype(np.float64), np.abs(r16.astype(np.float64))).max(axis=-1)
    es = e2m3.scale_exp(mx, -116)
    sc = np.exp2(es.astype(np.float64))[..., None]
    rec = np.zeros(pref.shape[:-1] + (64,), np.uint8)
    rec[..., :32] = p16.view(np.uint8).reshape(pref.shape[:-1] + (32,))
    rec[..., 32:44] = e2m3.pack16(e2m3.encode(p16.astype(np.float64) / sc))
    rec[..., 44:56] = e2m3.pack16(e2m3.encode(r16.astype(np.float64) / sc))
    rec[..., 56] = (116 + es).astype(np.uint8)
    return rec


def check_records(rec, pref, r_slack=0.05):
    """Assert that records [..., 64] encode the weights P' [..., 16] (float32
    references that may differ from the writer's own P' by ~2^-20 relative).
    P'16 within one fp16 ulp of fp16(P') (at most 1% of them off); the codes of
    P'16 exactly e2m3 of the record's own P'16 / 2^es; es the rule applied to
    the record's values (one larger only with a residual code of at least 3.5);
    the residual codes within half an e2m3 step (+ r_slack of the scale) of
    (P' - P'16) 2^11; zero padding."""
    rec = np.asarray(rec, np.uint8)
    pref = np.asarray(pref, np.float32)
    p16 = rec[..., :32].copy().view(np.float16).astype(np.float32).reshape(pref.shape)
    ref16 = pref.astype(np.float16).astype(np.float32)
    ulp = np.spacing(np.maximum(np.abs(ref16), np.float32(6.1e-5)).astype(np.float16)).astype(np.float32)
    off_by = np.abs(p16 - ref16) / ulp
    assert off_by.max() <= 1.0, ("P'16 off by more than one ulp", off_by.max())
    assert (off_by > 0).mean() < 0.01, ("P'16 off in too many places", (off_by > 0).mean())
    assert (rec[..., 57:64] == 0).all(), "padding bytes not zero"
    codes = e2m3.unpack16(rec[..., 32:44])
    rcodes = e2m3.unpack16(rec[..., 44:56])
    es = rec[..., 56].astype(np.int64) - 116
    sc = np.exp2(es.astype(np.float64))[..., None]
    assert (codes == e2m3.encode(p16.astype(np.float64) / sc)).all(), "codes of P'16"
    e1 = e2m3.scale_exp(p16.max(axis=-1), -116)
    rmag = np.abs(e2m3.decode(rcodes)).max(axis=-1)
    assert ((es == e1) | ((es == e1 + 1) & (rmag >= 3.5))).all(), "scale rule"
    r_ref = (pref.astype(np.float64) - p16) * 2048.0
    v = np.abs(r_ref) / sc
    step = np.where(v < 1.0, 1.0 / 8, np.exp2(np.floor(np.log2(np.maximum(v, 1.0)))) / 8)
    err = np.abs(e2m3.decode(rcodes) * sc - r_ref) / sc
    assert (err <= step / 2 + r_slack).all(), ("residual codes", (err - step / 2).max())
