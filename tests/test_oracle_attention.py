"""Pins for the oracle's bidirectional canvas attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle.attention import canvas_attention, canvas_attention_batched


def brute_force(q, kp, vp, kc, vc, scale):
    """Explicit loops: each query row against every prefix and canvas key."""
    n, hq, d = q.shape
    hkv = kc.shape[1]
    keys = list(kp) + list(kc)
    vals = list(vp) + list(vc)
    out = np.zeros((n, hq, d))
    for i in range(n):
        for h in range(hq):
            kvh = h // (hq // hkv)
            s = [scale * sum(q[i, h, t] * k[kvh, t] for t in range(d)) for k in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for t in range(d):
                out[i, h, t] = sum(w[j] * vals[j][kvh, t] for j in range(len(keys))) / tot
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    n, p, hq, hkv, d = 5, 7, 4, 2, 8
    q = rng.standard_normal((n, hq, d)); kp = rng.standard_normal((p, hkv, d))
    vp = rng.standard_normal((p, hkv, d)); kc = rng.standard_normal((n, hkv, d))
    vc = rng.standard_normal((n, hkv, d))
    got = canvas_attention(q, kp, vp, kc, vc)
    ref = brute_force(q, kp, vp, kc, vc, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,d,p", [(8, 8, 64, 256), (16, 8, 128, 96), (8, 2, 64, 0)])
def test_matches_torch_sdpa(hq, hkv, d, p):
    rng = np.random.default_rng(hq * 100 + p)
    n = 64
    q = rng.standard_normal((n, hq, d)); kp = rng.standard_normal((p, hkv, d))
    vp = rng.standard_normal((p, hkv, d)); kc = rng.standard_normal((n, hkv, d))
    vc = rng.standard_normal((n, hkv, d))
    got = canvas_attention(q, kp, vp, kc, vc)
    K = torch.from_numpy(np.concatenate([kp, kc])).permute(1, 0, 2)[None]
    V = torch.from_numpy(np.concatenate([vp, vc])).permute(1, 0, 2)[None]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = K.repeat_interleave(hq // hkv, dim=1)
    V = V.repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_closed_forms():
    rng = np.random.default_rng(3)
    n, hq, hkv, d = 6, 4, 2, 16
    q = rng.standard_normal((n, hq, d))
    kc = rng.standard_normal((n, hkv, d)); vc = rng.standard_normal((n, hkv, d))
    empty = np.zeros((0, hkv, d))
    # one key: the output is that key's value row
    o = canvas_attention(q[:1], empty, empty, kc[:1], vc[:1])
    for h in range(hq):
        np.testing.assert_allclose(o[0, h], vc[0, h // 2], atol=1e-14)
    # scale 0: uniform weights, the mean of the value rows
    o = canvas_attention(q, empty, empty, kc, vc, scale=0.0)
    for h in range(hq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(vc[:, h // 2].mean(0), (n, d)), atol=1e-13)
    # constant value rows: the output is that constant whatever the scores
    vconst = np.broadcast_to(rng.standard_normal((1, hkv, d)), (n, hkv, d))
    o = canvas_attention(q, empty, empty, kc, vconst)
    for h in range(hq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(vconst[0, h // 2], (n, d)), atol=1e-12)


def test_key_permutation_invariance_and_query_equivariance():
    q, kp, vp, kc, vc = workloads.attention_inputs(1, n=32, n_prefix=40, hq=4, hkv=2, head_dim=16)
    base = canvas_attention(q, kp, vp, kc, vc)
    rng = np.random.default_rng(7)
    pc = rng.permutation(kc.shape[0]); pp = rng.permutation(kp.shape[0])
    np.testing.assert_allclose(canvas_attention(q, kp, vp, kc[pc], vc[pc]), base, atol=1e-12)
    np.testing.assert_allclose(canvas_attention(q, kp[pp], vp[pp], kc, vc), base, atol=1e-12)
    pq = rng.permutation(q.shape[0])
    np.testing.assert_allclose(canvas_attention(q[pq], kp, vp, kc, vc), base[pq], atol=1e-12)


def test_gqa_mapping_is_blocked():
    # head h reads KV head h // G: giving KV head 1 zero values must zero heads 2, 3 only
    rng = np.random.default_rng(5)
    n, hq, hkv, d = 4, 4, 2, 8
    q = rng.standard_normal((n, hq, d)); kc = rng.standard_normal((n, hkv, d))
    vc = rng.standard_normal((n, hkv, d)); vc[:, 1] = 0
    o = canvas_attention(q, np.zeros((0, hkv, d)), np.zeros((0, hkv, d)), kc, vc)
    assert np.all(o[:, 2:] == 0) and np.all(np.abs(o[:, :2]) > 0)


@pytest.mark.parametrize("p", [0, 40])
def test_causal_matches_torch_sdpa_with_mask(p):
    """Causal flag: canvas row i sees the prefix and canvas keys 0..i (torch's SDPA
    with an explicit boolean mask is the independent routine)."""
    rng = np.random.default_rng(70 + p)
    n, hq, hkv, d = 48, 8, 4, 64
    q = rng.standard_normal((n, hq, d)); kp = rng.standard_normal((p, hkv, d))
    vp = rng.standard_normal((p, hkv, d)); kc = rng.standard_normal((n, hkv, d))
    vc = rng.standard_normal((n, hkv, d))
    got = canvas_attention(q, kp, vp, kc, vc, causal=True)
    K = torch.from_numpy(np.concatenate([kp, kc])).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    V = torch.from_numpy(np.concatenate([vp, vc])).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    allowed = np.ones((n, p + n), dtype=bool)
    allowed[:, p:] = np.tril(np.ones((n, n), dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(allowed))[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_causal_special_cases():
    rng = np.random.default_rng(71)
    n, p, hq, hkv, d = 20, 9, 4, 4, 16
    q = rng.standard_normal((n, hq, d)); kp = rng.standard_normal((p, hkv, d))
    vp = rng.standard_normal((p, hkv, d)); kc = rng.standard_normal((n, hkv, d))
    vc = rng.standard_normal((n, hkv, d))
    full = canvas_attention(q, kp, vp, kc, vc)
    causal = canvas_attention(q, kp, vp, kc, vc, causal=True)
    # the last canvas row sees every key either way
    np.testing.assert_allclose(causal[-1], full[-1], rtol=1e-13, atol=1e-13)
    # with no prefix, canvas row 0 sees only its own key: O = v_0
    c0 = canvas_attention(q, None, None, kc, vc, causal=True)
    np.testing.assert_allclose(c0[0], vc[0], rtol=1e-13, atol=1e-13)
    # row i does not depend on canvas keys after i
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[10:] = rng.standard_normal((n - 10, hkv, d)); vc2[10:] = 5.0
    c2 = canvas_attention(q, kp, vp, kc2, vc2, causal=True)
    np.testing.assert_allclose(c2[:10], causal[:10], rtol=1e-13, atol=1e-13)


def test_batched_matches_torch_sdpa_over_the_padded_layout():
    """A batch of sequences with ragged prefixes and mixed causal flags: torch's
    SDPA over the padded [prefix slab ; canvas] layout with a boolean mask that
    hides each sequence's padding rows, and its later canvas keys where the flag
    is set.  Padding holds large finite values, so any leak would show."""
    rng = np.random.default_rng(90)
    b, n, stride, hq, hkv, d = 4, 24, 30, 8, 2, 32
    nps, flags = [30, 0, 17, 5], [False, True, True, False]
    q = rng.standard_normal((b, n, hq, d))
    kp = rng.standard_normal((b, stride, hkv, d)); vp = rng.standard_normal((b, stride, hkv, d))
    kc = rng.standard_normal((b, n, hkv, d)); vc = rng.standard_normal((b, n, hkv, d))
    for s_, np_s in enumerate(nps):
        kp[s_, np_s:] = 1e3; vp[s_, np_s:] = -1e3
    got = canvas_attention_batched(q, kp, vp, kc, vc, nps, flags)
    K = torch.from_numpy(np.concatenate([kp, kc], axis=1)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    V = torch.from_numpy(np.concatenate([vp, vc], axis=1)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    allowed = np.zeros((b, 1, n, stride + n), dtype=bool)
    for s_, (np_s, c) in enumerate(zip(nps, flags)):
        allowed[s_, 0, :, :np_s] = True
        allowed[s_, 0, :, stride:] = np.tril(np.ones((n, n), dtype=bool)) if c else True
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(allowed)).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_batched_sequences_are_independent():
    """Sequence 0's output depends neither on sequence 1's inputs nor on its own
    padding rows; sequence 1's output does change with its inputs."""
    rng = np.random.default_rng(91)
    b, n, stride, hq, hkv, d = 2, 16, 20, 4, 4, 16
    nps, flags = [11, 20], [True, False]
    q = rng.standard_normal((b, n, hq, d))
    kp = rng.standard_normal((b, stride, hkv, d)); vp = rng.standard_normal((b, stride, hkv, d))
    kc = rng.standard_normal((b, n, hkv, d)); vc = rng.standard_normal((b, n, hkv, d))
    o1 = canvas_attention_batched(q, kp, vp, kc, vc, nps, flags)
    q2, kp2, vp2, kc2 = q.copy(), kp.copy(), vp.copy(), kc.copy()
    q2[1] += 1.0; kc2[1] *= -1.0; kp2[1, 3] += 2.0
    kp2[0, nps[0]:] = np.nan; vp2[0, nps[0]:] = np.inf
    o2 = canvas_attention_batched(q2, kp2, vp2, kc2, vc, nps, flags)
    assert np.array_equal(o1[0], o2[0])
    assert not np.allclose(o1[1], o2[1])
    # each sequence is the single-sequence definition with its own flag
    np.testing.assert_array_equal(o1[0], canvas_attention(q[0], kp[0, :11], vp[0, :11], kc[0], vc[0], causal=True))
