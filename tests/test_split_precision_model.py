"""The packed contraction's number format, modelled on the CPU (no GPU, no
library code): z = softmax(l)·E computed with the roundings the packed path
makes, against the fp64 product.

The sampler must give z at full precision (DiffusionGemma Technical Report part
4/6, section 6 "Sampling"); the parity bound is relative L2 1e-4.  The packed
path holds P = 2^14·p and Q = 2^c·E (max|Q| in [2^7, 2^8)) as fp16 plus e4m3
corrections and sums, per term,
    P16·Q16 + 2^-5·[ fp8(P·2^-6)·fp8((Q - Q16)·2^11) + fp8((P - P16)·2^5)·fp8(Q16) ].
Here fp16 rounding is numpy's and e4m3 rounding is torch's float8_e4m3fn
(round to nearest even), the roundings the GPU's conversions make (fp32 to
fp16 and to e4m3 are compared byte for byte in
tests/test_gpu_sampler.py::test_embedding_pack_layout).  The test shows two
things:
  - the format meets the bound with a wide margin on varied rows and tables;
  - the bound rejects the plausible mistakes: either correction term dropped,
    both dropped (fp16 alone), or the wrong block scale on the corrections.
"""
import math

import numpy as np
import pytest
import torch

V, D = 65536, 64
BOUND = 1e-4


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def _f8(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _model(logits, emb, variant="exact"):
    """z rows with the packed format's roundings; variant plants one mistake."""
    e = math.frexp(float(np.abs(emb).max()))[1]
    c = min(8 - e, 80)
    q = (emb.astype(np.float32) * np.float32(2.0 ** c)).astype(np.float32)
    q16 = _f16(q)
    qe8 = _f8((q - q16.astype(np.float32)) * np.float32(2048.0))
    q8 = _f8(q16.astype(np.float32))
    scale = 2.0 ** -4 if variant == "scale" else 2.0 ** -5
    rows = []
    for l in logits:
        p = np.exp2(((l - l.max()) * np.float32(math.log2(math.e))).astype(np.float32)).astype(np.float32)
        big_p = (p * np.float32(16384.0)).astype(np.float32)
        p16 = _f16(big_p)
        pe8 = _f8((big_p - p16.astype(np.float32)) * np.float32(32.0))
        p8 = _f8(big_p * np.float32(1.0 / 64.0))
        acc = p16 @ q16
        if variant not in ("no_pqe", "fp16"):
            acc += scale * (p8 @ qe8)
        if variant not in ("no_peq", "fp16"):
            acc += scale * (pe8 @ q8)
        rows.append(acc / p.astype(np.float64).sum() * 2.0 ** -(14 + c))
    return np.array(rows)


def _exact(logits, emb):
    rows = []
    for l in logits:
        w = np.exp(l.astype(np.float64) - float(l.max()))
        rows.append(w @ emb.astype(np.float64) / w.sum())
    return np.array(rows)


def _inputs(scale):
    rng = np.random.default_rng(int(scale * 1e6) % 1000 + 7)
    emb = (rng.standard_normal((V, D)) * scale).astype(np.float32)
    logits = np.stack([rng.standard_normal(V) * s for s in (1.0, 3.0, 0.3)]).astype(np.float32)
    logits[1, 77] += 12.0                      # one dominant id
    return logits, emb


def _rel(z, ref):
    return np.array([np.linalg.norm(a - b) / np.linalg.norm(b) for a, b in zip(z, ref)])


@pytest.mark.parametrize("scale", [0.02, 300.0, 1e-5])
def test_packed_format_meets_the_bound(scale):
    logits, emb = _inputs(scale)
    rel = _rel(_model(logits, emb), _exact(logits, emb))
    assert rel.max() < BOUND / 4, rel


@pytest.mark.parametrize("variant", ["no_pqe", "no_peq", "fp16", "scale"])
def test_bound_rejects_a_planted_mistake(variant):
    logits, emb = _inputs(0.02)
    ref = _exact(logits, emb)
    good = _rel(_model(logits, emb), ref)
    bad = _rel(_model(logits, emb, variant), ref)
    assert good.max() < BOUND / 4
    assert bad.max() > BOUND, (variant, bad)
