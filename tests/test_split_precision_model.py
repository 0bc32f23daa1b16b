"""The packed contraction's number format, modelled on the CPU (no GPU, no
library code): z = softmax(l)·E computed with the roundings the packed path
makes, against the fp64 product.

The sampler must give z at full precision (DiffusionGemma Technical Report part
4/6, section 6 "Sampling"); the parity bound is relative L2 1e-4.  The packed
path holds the table as Q_k = E_k·2^(c + d_k): c brings max|E| to [2^7, 2^8)
and the row shift d_k (at most 40; 40 for zero rows) brings row k's own
maximum there too.  The weights carry the inverse shift, P'_k = p_k·2^(14 - d_k),
so that P'_k·Q_k = 2^(14 + c)·p_k·E_k.  With fp16 P'16, Q16 the product is
    P'16·Q16 + P'16·(Q - Q16) + (P' - P'16)·Q16,
the last two terms in e2m3 (fp6) under power-of-two block scales:
  - per row and 16-id k-block, the codes of P'16 and of r = fp16((P' - P'16)·2^11),
    divided by 2^es, the smallest power of two (at least 2^-116) bringing the
    block's largest value to 7.5 or below; the matrix core applies 2^(es - 11);
  - per 16-id k-block and 64-column group, the codes of (Q - Q16)·2^11 and of
    Q16 under one scale 2^eB (at least 2^-126).
fp16 rounding is numpy's; e2m3 rounding (nearest, ties to the even code) is
tests/e2m3.py's, the rounding of the GPU's conversions (the table's codes are
compared byte for byte in tests/test_gpu_sampler.py::test_embedding_pack_layout).
The test shows:
  - the format meets the bound with a margin on varied rows and tables,
    including tables whose rows differ in size by up to 2^60;
  - the bound rejects the plausible mistakes: either correction term dropped,
    both dropped (fp16 alone), the wrong factor on the corrections, no row
    shifts (one block scale over rows of very different size), and zero rows
    left unshifted (their weights set the k-block's scale).
"""
import math

import numpy as np
import pytest

import e2m3

BOUND = 1e-4


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def _table(emb, variant):
    """Padded table values: c, row shifts d, Q16 and the decoded corrections."""
    v0, d0 = emb.shape
    v, d = -(-v0 // 16) * 16, -(-d0 // 64) * 64
    full = np.zeros((v, d), np.float32)
    full[:v0, :d0] = emb
    c = min(8 - math.frexp(float(np.abs(emb).max()))[1], 80)
    m = np.abs(full).max(axis=1).astype(np.float64)
    shift = np.where(m > 0, np.clip(8 - c - np.frexp(m)[1], 0, 40), 40)
    if variant == "no_shift":
        shift[:] = 0
    if variant == "zero_rows_unshifted":
        shift[m == 0] = 0
    q = full * np.exp2(c + shift)[:, None].astype(np.float32)         # exact power-of-two scaling
    q16 = _f16(q)
    qe = ((q - q16.astype(np.float32)) * np.float32(2048.0)).astype(np.float64)
    nb, ng = v // 16, d // 64
    mx = np.maximum(np.abs(qe), np.abs(q16)).reshape(nb, 16, ng, 64).max(axis=(1, 3))
    sb = np.exp2(e2m3.scale_exp(mx, -126))[:, None, :, None]
    dq = lambda x: (e2m3.decode(e2m3.encode(x.reshape(nb, 16, ng, 64) / sb)) * sb).reshape(v, d)
    return c, shift, q16, dq(qe), dq(q16)


def _model(logits, emb, variant="exact"):
    """z rows with the packed format's roundings; variant plants one mistake."""
    v0, d0 = emb.shape
    c, shift, q16, qe6, q6 = _table(emb, variant)
    v = q16.shape[0]
    nb = v // 16
    factor = 2.0 ** -10 if variant == "scale" else 2.0 ** -11
    rows = []
    for l in logits:
        lf = np.full(v, -np.inf, np.float32)
        lf[:v0] = l
        p = np.exp2(((lf - l.max()) * np.float32(math.log2(math.e))).astype(np.float32)).astype(np.float32)
        big_p = np.ldexp(p, (14 - shift).astype(np.int32)).astype(np.float32)            # P', exact
        p16 = _f16(big_p)
        r16 = _f16((big_p - p16.astype(np.float32)) * np.float32(2048.0))
        mx = np.maximum(p16, np.abs(r16)).reshape(nb, 16).max(axis=1)
        sa = np.exp2(e2m3.scale_exp(mx, -116))[:, None]
        p6 = (e2m3.decode(e2m3.encode(p16.reshape(nb, 16) / sa)) * sa).reshape(v) * factor
        r6 = (e2m3.decode(e2m3.encode(r16.reshape(nb, 16) / sa)) * sa).reshape(v) * factor
        acc = p16 @ q16
        if variant not in ("no_pqe", "fp16"):
            acc += p6 @ qe6
        if variant not in ("no_peq", "fp16"):
            acc += r6 @ q6
        rows.append((acc / p.astype(np.float64).sum() * 2.0 ** -(14 + c))[:d0])
    return np.array(rows)


def _exact(logits, emb):
    rows = []
    for l in logits:
        w = np.exp(l.astype(np.float64) - float(l.max()))
        rows.append(w @ emb.astype(np.float64) / w.sum())
    return np.array(rows)


def _inputs(scale):
    rng = np.random.default_rng(int(scale * 1e6) % 1000 + 7 + (3 if scale < 1e-20 else 0))
    emb = (rng.standard_normal((65536, 64)) * scale).astype(np.float32)
    logits = np.stack([rng.standard_normal(65536) * s for s in (1.0, 3.0, 0.3)]).astype(np.float32)
    logits[1, 77] += 12.0                      # one dominant id
    return logits, emb


def _outlier_inputs():
    """one row near 1 among rows of 0.02: the outlier shares k-blocks with small rows"""
    rng = np.random.default_rng(2)
    n, vocab, d = 32, 29, 40
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::4, vocab - 1] += 9.0
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb[vocab - 1] += 1.0
    return logits, emb


def _spread_inputs(spread):
    """rows scaled by 2^u, u in [-spread, 0], every 16th row 2^spread larger, some rows zero"""
    rng = np.random.default_rng(spread)
    n, vocab, d = 96, 4099, 200
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb *= np.exp2(rng.uniform(-spread, 0, vocab))[:, None].astype(np.float32)
    emb[::16] *= np.float32(2.0 ** spread)
    emb[5::23] = 0.0
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::5, 17] += 8.0
    return logits, emb


def _rel(z, ref):
    return np.array([np.linalg.norm(a - b) / np.linalg.norm(b) for a, b in zip(z, ref)])


@pytest.mark.parametrize("scale", [0.02, 300.0, 1e-5, 1e-25])
def test_packed_format_meets_the_bound(scale):
    logits, emb = _inputs(scale)
    rel = _rel(_model(logits, emb), _exact(logits, emb))
    assert rel.max() < BOUND / 3, rel


@pytest.mark.parametrize("case", ["outlier", "spread6", "spread30"])
def test_packed_format_meets_the_bound_on_uneven_rows(case):
    logits, emb = _outlier_inputs() if case == "outlier" else _spread_inputs(int(case[6:]))
    rel = _rel(_model(logits, emb), _exact(logits, emb))
    assert rel.max() < BOUND / 2, rel


@pytest.mark.parametrize("variant,case", [("no_pqe", "plain"), ("no_peq", "plain"), ("fp16", "plain"),
                                          ("scale", "plain"), ("no_shift", "outlier"),
                                          ("zero_rows_unshifted", "spread30")])
def test_bound_rejects_a_planted_mistake(variant, case):
    logits, emb = {"plain": lambda: _inputs(0.02), "outlier": _outlier_inputs,
                   "spread30": lambda: _spread_inputs(30)}[case]()
    ref = _exact(logits, emb)
    good = _rel(_model(logits, emb), ref)
    bad = _rel(_model(logits, emb, variant), ref)
    assert good.max() < BOUND / 2
    assert bad.max() > BOUND, (variant, bad.max())
