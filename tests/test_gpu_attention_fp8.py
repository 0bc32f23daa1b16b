"""FP8 (OCP E4M3) canvas attention on the GPU against the oracle: attention of
the decoded, scaled inputs in fp64 (oracle.fp8).  The kernel stages E4M3 as
bf16 exactly, so the bf16 path's bounds apply to the decoded, scaled inputs:
max-abs 2e-2 on outputs of unit-scale values (scaled by v_scale) and the
secondary rounding bounds of tests/gpu_util.py."""
import numpy as np
import pytest

import workloads
from gpu_util import ATTN_MAX_ABS, ATTN_ROW_REL, attention_errors, attention_reference, log, require_gpu, to_dev
from oracle import fp8 as F

pytestmark = pytest.mark.gpu


def run_fp8(torch, dg, q, kp, vp, kc, vc, scales=(1.0, 1.0, 1.0), causal=False):
    tq, tkc, tvc = to_dev(q), to_dev(kc), to_dev(vc)
    tkp = to_dev(kp) if kp.shape[0] else None
    tvp = to_dev(vp) if kp.shape[0] else None
    out = dg.dg_canvas_attention_fp8(tq, tkp, tvp, tkc, tvc, *scales, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, codes, scales, label, tol, causal=False):
    """The contract (tol) and the secondary bounds around the oracle on the
    decoded, scaled inputs (the kernel stages them exactly)."""
    q, kp, vp, kc, vc = codes
    qs, ks, vs = scales
    dq = lambda x, sc: F.e4m3_to_float(x) * float(np.float32(sc))
    ref = F.canvas_attention_fp8(q, kp, vp, kc, vc, *scales, causal=causal)
    _, ref_r, bound = attention_reference(dq(q, qs), dq(kp, ks), dq(vp, vs), dq(kc, ks), dq(vc, vs), causal=causal,
                                          scale=1.0 / np.sqrt(q.shape[2]))
    assert np.all(np.isfinite(got))
    err, ratio, row = attention_errors(got, ref, ref_r, bound)
    log(f"{label}: max abs err {err:.3e}, error / element bound {ratio:.3f}, row rel L2 {row:.3e}")
    assert err <= tol, f"{label}: max abs err {err}"
    assert ratio <= 1.0, f"{label}: error exceeds the rounding bound by {ratio:.2f}x"
    assert row <= ATTN_ROW_REL, f"{label}: row relative L2 {row:.3e}"


def test_long_context_fp8_with_scales():
    torch, dg = require_gpu()
    q, kp, vp, kc, vc = workloads.attention_inputs_fp8(4)
    scales = (0.5, 0.75, 2.0)
    got = run_fp8(torch, dg, q, kp, vp, kc, vc, scales)
    check(got, (q, kp, vp, kc, vc), scales, "long context, fp8", ATTN_MAX_ABS * scales[2])


@pytest.mark.parametrize("n,p,hq,hkv,d,causal", [
    (256, 0, 16, 8, 128, False),
    (100, 37, 16, 8, 128, False),
    (130, 300, 8, 2, 64, False),
    (1, 5, 8, 8, 64, False),
    (256, 512, 16, 8, 128, True),
    (77, 130, 16, 4, 64, True),
    (64, 0, 16, 8, 128, False),        # one key block: a single chunk, output written directly
])
def test_fp8_shapes(n, p, hq, hkv, d, causal):
    torch, dg = require_gpu()
    log(f"fp8 attention n={n} p={p} hq={hq} hkv={hkv} d={d} causal={causal}")
    q, kp, vp, kc, vc = workloads.attention_inputs_fp8(2, n=n, n_prefix=p, hq=hq, hkv=hkv, head_dim=d)
    got = run_fp8(torch, dg, q, kp, vp, kc, vc, causal=causal)
    check(got, (q, kp, vp, kc, vc), (1.0, 1.0, 1.0), f"n={n} p={p}", ATTN_MAX_ABS, causal=causal)


def test_every_code_decodes_exactly():
    """Zero keys give equal weights (exactly 1 each on the device), so O is the
    mean of the decoded values; one 64-key block means one chunk and an fp32
    output straight from the registers.  Every finite code appears in V."""
    torch, dg = require_gpu()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n, d = 64, 64
    vc = np.stack([np.roll(codes, -4 * j)[:d] for j in range(n)])[:, None, :]    # [64, 1, 64]
    assert set(np.unique(vc).tolist()) == set(codes.tolist())
    kc = np.zeros((n, 1, d), np.uint8)
    empty = np.zeros((0, 1, d), np.uint8)
    q = workloads.fp8_codes(np.random.default_rng(0).standard_normal((n, 1, d)))
    got = run_fp8(torch, dg, q, empty, empty, kc, vc)
    ref = F.canvas_attention_fp8(q, empty, empty, kc, vc)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-3)


def every_code_inputs(d):
    """Q row i holds one nonzero E4M3 code, at element i, and key j holds code
    (3j + 5c) mod 254 of the finite codes at element c, so score (i, j) is the
    single product q_i * k_j[i]: exact in float32 whatever the accumulation
    order, and every finite code of K (subnormals, zeros, +-448) meets the FP8
    matrix cores.  V is the identity, so O row i is query i's weight vector."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = d
    q = np.zeros((n, 1, d), np.uint8)
    for i in range(n):
        q[i, 0, i] = codes[(7 * i + 3) % len(codes)]
    j, c = np.meshgrid(np.arange(n), np.arange(d), indexing="ij")
    kc = codes[(3 * j + 5 * c) % len(codes)][:, None, :]
    eye = workloads.fp8_codes(np.eye(n, d, dtype=np.float32))[:, None, :]
    return q, kc, eye, codes


@pytest.mark.parametrize("d", [64, 128])
def test_every_code_through_the_fp8_scores(d):
    """The FP8 matrix-core scores, element by element: O = the softmax weights
    of exact single-product scores (scale 1/64), against the oracle on the
    decoded codes.  Each weight is rounded to bf16 for the P.V product (unit
    roundoff 2^-8) and divided by the float32 sum: (2^-8 + 2^-11) relative, the
    second term for the exponent and sum roundings, plus float32 noise, bounds
    the difference."""
    torch, dg = require_gpu()
    log(f"fp8 scores over every code, d={d}")
    q, kc, eye, codes = every_code_inputs(d)
    assert set(np.unique(kc).tolist()) == set(codes.tolist())
    empty = np.zeros((0, 1, d), np.uint8)
    out = dg.dg_canvas_attention_fp8(to_dev(q), None, None, to_dev(kc), to_dev(eye), scale=1.0 / 64)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = F.canvas_attention_fp8(q, empty, empty, kc, eye, scale=1.0 / 64)
    err = np.abs(got - ref)
    worst = float((err / ((2.0 ** -8 + 2.0 ** -11) * np.abs(ref) + 1e-6)).max())
    log(f"every code, d={d}: worst error / ((2^-8 + 2^-11) |w| + 1e-6) = {worst:.3f}")
    assert worst <= 1.0
