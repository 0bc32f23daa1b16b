"""The secondary attention bound (tests/gpu_util.py) against planted mistakes, on
the CPU: a model of the kernel's bf16 rounding of P passes it with a wide
margin, while a mistake of the size a mask, tail or head-map bug makes fails it,
even where the 2e-2 contract alone would not notice."""
import numpy as np
import pytest

import workloads
from gpu_util import ATTN_MAX_ABS, ATTN_ROW_REL, attention_errors, attention_reference
from oracle.attention import canvas_attention


def rounded_p_model(q, kp, vp, kc, vc, group):
    """Softmax weights in float64, P rounded to bf16 for the P.V product and the
    sum taken over the unrounded P: the roundings the element bound assumes."""
    keys = np.concatenate([kp, kc]).astype(np.float64)
    vals = np.concatenate([vp, vc]).astype(np.float64)
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        s = q[:, h, :].astype(np.float64) @ keys[:, h // group, :].T / np.sqrt(q.shape[2])
        w = np.exp(s - s.max(axis=1, keepdims=True))
        pb = workloads.round_bf16(w.astype(np.float32)).astype(np.float64)
        out[:, h, :] = pb @ vals[:, h // group, :] / w.sum(axis=1, keepdims=True)
    return out


@pytest.fixture(scope="module")
def long_context():
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    ref, ref_r, bound = attention_reference(q, kp, vp, kc, vc)
    return (q, kp, vp, kc, vc), ref, ref_r, bound


def test_rounding_model_is_well_inside(long_context):
    (q, kp, vp, kc, vc), ref, ref_r, bound = long_context
    err, ratio, row = attention_errors(rounded_p_model(q, kp, vp, kc, vc, 2), ref, ref_r, bound)
    assert err < ATTN_MAX_ABS / 20
    assert ratio < 0.25
    assert row < ATTN_ROW_REL / 2


def drop_key(q, kp, vp, kc, vc, key):
    """The oracle with one key of the [prefix ; canvas] sequence hidden from every row."""
    keys = np.concatenate([kp, kc]).astype(np.float64)
    vals = np.concatenate([vp, vc]).astype(np.float64)
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        s = q[:, h, :].astype(np.float64) @ keys[:, h // 2, :].T / np.sqrt(q.shape[2])
        s[:, key] = -np.inf
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ vals[:, h // 2, :]
    return out


@pytest.mark.parametrize("key", [4095, 4096, 4351, 64 * 17])   # block edges of the prefix and the canvas
def test_one_dropped_key_fails_the_bound(long_context, key):
    (q, kp, vp, kc, vc), ref, ref_r, bound = long_context
    err, ratio, row = attention_errors(drop_key(q, kp, vp, kc, vc, key), ref, ref_r, bound)
    assert err <= ATTN_MAX_ABS          # the contract alone lets it through
    assert ratio > 1.5 and row > 5 * ATTN_ROW_REL


def test_head_map_and_mask_mistakes_fail_the_bound():
    q, kp, vp, kc, vc = workloads.attention_inputs(2, n=64, n_prefix=200, hq=16, hkv=4)
    ref, ref_r, bound = attention_reference(q, kp, vp, kc, vc)
    # kv = h % Hkv instead of h // (Hq / Hkv)
    swapped = q.reshape(64, 4, 4, 128).transpose(0, 2, 1, 3).reshape(64, 16, 128)
    wrong = canvas_attention(swapped, kp, vp, kc, vc).reshape(64, 4, 4, 128).transpose(0, 2, 1, 3)
    assert attention_errors(wrong.reshape(64, 16, 128), ref, ref_r, bound)[1] > 10
    # a causal off-by-one: canvas row i also sees key i + 1
    ref_c, ref_cr, bound_c = attention_reference(q, kp, vp, kc, vc, causal=True)
    leak = np.empty_like(ref_c)
    for i in range(64):
        j = min(i + 2, 64)
        leak[i] = canvas_attention(q[i:i + 1], np.concatenate([kp, kc[:i]]), np.concatenate([vp, vc[:i]]),
                                   kc[i:j], vc[i:j])[0]
    _, ratio, row = attention_errors(leak, ref_c, ref_cr, bound_c)
    assert ratio > 1.5 and row > ATTN_ROW_REL


def test_staged_fp32_inputs_use_the_rounded_reference():
    """Float32 inputs are rounded to bf16 when staged: the bound sits around the
    oracle on the rounded inputs.  The input rounding alone moves the output by
    a sizeable part of the bound (about half of it at head_dim 64), which the
    bound would otherwise have to absorb, and the rounded-P model of the kernel
    stays well inside the bound around the rounded reference."""
    q, kp, vp, kc, vc = workloads.attention_inputs(1, n=64, n_prefix=64)
    ref, ref_r, bound = attention_reference(q, kp, vp, kc, vc, staged_bf16=True)
    assert np.abs(ref_r - ref).max() < ATTN_MAX_ABS
    assert (np.abs(ref_r - ref) / bound).max() > 0.2
    r = [workloads.round_bf16(t) for t in (q, kp, vp, kc, vc)]
    assert attention_errors(rounded_p_model(*r, 1), ref, ref_r, bound)[1] < 0.25
