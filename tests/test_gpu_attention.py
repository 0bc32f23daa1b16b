"""Canvas attention on the GPU against the fp64 oracle: the max-abs 2e-2 contract (bf16 in,
fp32 accumulate) and the secondary rounding bounds (element and row) of tests/gpu_util.py."""
import numpy as np
import pytest

import workloads
from gpu_util import ATTN_MAX_ABS, attention_reference, check_attention, log, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(torch, dg, q, kp, vp, kc, vc, qkv, scale=0.0):
    dt = torch.bfloat16 if qkv == "bf16" else torch.float32
    tq, tkc, tvc = to_dev(q, dt), to_dev(kc, dt), to_dev(vc, dt)
    tkp = to_dev(kp, dt) if kp.shape[0] else None
    tvp = to_dev(vp, dt) if kp.shape[0] else None
    out = dg.dg_canvas_attention(tq, tkp, tvp, tkc, tvc, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, inputs, label, qkv="bf16", causal=False, scale=None):
    """The contract and the secondary bounds against the oracle on these inputs."""
    ref, ref_r, bound = attention_reference(*inputs, causal=causal, scale=scale, staged_bf16=(qkv == "f32"))
    return check_attention(got, ref, ref_r, bound, label)


@pytest.mark.parametrize("workload", [1, 2, 4])
def test_workloads(workload):
    torch, dg = require_gpu()
    c = workloads.CONFIGS[workload]
    log(f"attention workload {workload}")
    q, kp, vp, kc, vc = workloads.attention_inputs(workload)
    got = run_gpu(torch, dg, q, kp, vp, kc, vc, c["qkv"])
    check(got, (q, kp, vp, kc, vc), f"workload {workload}", qkv=c["qkv"])


@pytest.mark.parametrize("n,p,hq,hkv,d,qkv", [
    (256, 0, 16, 8, 128, "bf16"),      # no prefix: canvas only
    (100, 37, 16, 8, 128, "bf16"),     # ragged query tile and ragged key block
    (1, 5, 8, 8, 64, "bf16"),          # a single canvas position
    (64, 200, 16, 4, 128, "bf16"),     # group of 4 query heads per KV head
    (130, 300, 8, 2, 64, "f32"),       # fp32 inputs staged as bf16, D=64, ragged
    (256, 5120, 16, 8, 128, "bf16"),   # largest prefix of the decode run
    (64, 0, 16, 8, 128, "bf16"),       # one key block in all: one chunk, output written directly
    (40, 0, 8, 2, 64, "f32"),          # the same single-chunk path at D=64, ragged block
    (64, 2048, 4, 2, 64, "bf16"),      # 33 key chunks: the merge beyond its 16-chunk one-pass form
])
def test_shapes(n, p, hq, hkv, d, qkv):
    torch, dg = require_gpu()
    log(f"attention n={n} p={p} hq={hq} hkv={hkv} d={d} {qkv}")
    q, kp, vp, kc, vc = workloads.attention_inputs(2, n=n, n_prefix=p, hq=hq, hkv=hkv, head_dim=d, qkv=qkv)
    got = run_gpu(torch, dg, q, kp, vp, kc, vc, qkv)
    check(got, (q, kp, vp, kc, vc), f"n={n} p={p}", qkv=qkv)


def test_explicit_scale():
    torch, dg = require_gpu()
    q, kp, vp, kc, vc = workloads.attention_inputs(2, n=64, n_prefix=64)
    got = run_gpu(torch, dg, q, kp, vp, kc, vc, "bf16", scale=0.05)
    check(got, (q, kp, vp, kc, vc), "scale 0.05", scale=0.05)


def test_permutation_invariance_and_equivariance():
    torch, dg = require_gpu()
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    base = run_gpu(torch, dg, q, kp, vp, kc, vc, "bf16")
    rng = np.random.default_rng(3)
    pc = rng.permutation(kc.shape[0])
    permuted = run_gpu(torch, dg, q, kp, vp, kc[pc], vc[pc], "bf16")
    assert np.abs(permuted - base).max() <= ATTN_MAX_ABS
    check(permuted, (q, kp, vp, kc[pc], vc[pc]), "permuted canvas keys")
    pq = rng.permutation(q.shape[0])
    # query rows are independent: permuting queries permutes the output exactly
    np.testing.assert_array_equal(run_gpu(torch, dg, q[pq], kp, vp, kc, vc, "bf16"), base[pq])


def test_deterministic():
    torch, dg = require_gpu()
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    a = run_gpu(torch, dg, q, kp, vp, kc, vc, "bf16")
    b = run_gpu(torch, dg, q, kp, vp, kc, vc, "bf16")
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("n,p,hq,hkv,d,qkv", [
    (256, 4096, 16, 8, 128, "bf16"),   # the KV-update pass at the long-context shape
    (256, 0, 16, 8, 128, "bf16"),      # no prefix: row 0 sees only its own key
    (100, 37, 16, 8, 128, "bf16"),     # ragged tiles and blocks
    (130, 300, 8, 2, 64, "f32"),       # fp32 inputs, D=64
    (1, 5, 8, 8, 64, "bf16"),          # a single canvas position
    (64, 0, 16, 8, 128, "bf16"),       # single chunk: the direct-output path with the causal mask
])
def test_causal(n, p, hq, hkv, d, qkv):
    torch, dg = require_gpu()
    log(f"causal attention n={n} p={p} hq={hq} hkv={hkv} d={d} {qkv}")
    q, kp, vp, kc, vc = workloads.attention_inputs(2, n=n, n_prefix=p, hq=hq, hkv=hkv, head_dim=d, qkv=qkv)
    dt = torch.bfloat16 if qkv == "bf16" else torch.float32
    t = lambda x: to_dev(x, dt)
    got = dg.dg_canvas_attention(t(q), t(kp) if p else None, t(vp) if p else None, t(kc), t(vc),
                                 causal=True).cpu().numpy()
    check(got, (q, kp, vp, kc, vc), f"causal n={n} p={p}", qkv=qkv, causal=True)


def batched_inputs(qkv, n, stride, nps, hq, hkv, d):
    """Per-sequence inputs in the padded batch layout; the prefix padding rows
    are NaN, so a read of them would show in the output.  Each prefix is rolled
    along the head dimension by its own amount, so equal-length prefixes differ."""
    b = len(nps)
    q = np.zeros((b, n, hq, d), np.float32)
    kc = np.zeros((b, n, hkv, d), np.float32)
    vc = np.zeros((b, n, hkv, d), np.float32)
    kp = np.full((b, stride, hkv, d), np.nan, np.float32)
    vp = np.full((b, stride, hkv, d), np.nan, np.float32)
    for s_, np_s in enumerate(nps):
        qs, kps, vps, kcs, vcs = workloads.attention_inputs(2, n=n, n_prefix=np_s, hq=hq, hkv=hkv, head_dim=d,
                                                             qkv=qkv, block=s_)
        q[s_], kc[s_], vc[s_] = qs, kcs, vcs
        kp[s_, :np_s] = np.roll(kps, 5 * s_, axis=-1)
        vp[s_, :np_s] = np.roll(vps, 3 * s_, axis=-1)
    return q, kp, vp, kc, vc


@pytest.mark.parametrize("qkv,n,stride,nps,flags,hq,hkv,d", [
    ("bf16", 256, 320, [100, 0, 320], [0, 1, 0], 16, 8, 128),             # ragged prefixes, one empty
    ("f32", 40, 130, [130, 7], [1, 0], 8, 2, 64),                          # fp32 staged, D=64, empty key chunks
    ("bf16", 256, 512, [512, 0, 64, 257, 511, 1, 300, 128],
     [0, 1, 0, 1, 1, 0, 0, 1], 16, 8, 128),                                # one chunk per sequence: direct output
    ("bf16", 256, 4096, [4096, 4096, 2048, 0], [0, 1, 0, 1], 16, 8, 128),  # long context, both pass types
])
def test_batched_mixed_causal(qkv, n, stride, nps, flags, hq, hkv, d):
    """Denoising (bidirectional) and KV-update (causal) passes of different
    sequences in one launch, each against the oracle's per-sequence definition."""
    torch, dg = require_gpu()
    log(f"batched attention nps={nps} causal={flags} n={n} stride={stride} hq={hq} hkv={hkv} d={d} {qkv}")
    q, kp, vp, kc, vc = batched_inputs(qkv, n, stride, nps, hq, hkv, d)
    dt = torch.bfloat16 if qkv == "bf16" else torch.float32
    out = dg.dg_canvas_attention_batched(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt), to_dev(kc, dt),
                                         to_dev(vc, dt), nps, [bool(f) for f in flags])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for s_ in range(len(nps)):
        np_s = nps[s_]
        check(got[s_], (q[s_], kp[s_, :np_s], vp[s_, :np_s], kc[s_], vc[s_]),
              f"sequence {s_} (n_prefix {np_s}, causal {flags[s_]})", qkv=qkv, causal=bool(flags[s_]))


def test_batched_single_sequence_matches_the_single_call():
    """A batch of one runs the same kernels with the same plan: bit-identical."""
    torch, dg = require_gpu()
    log("batched attention, batch of one against dg_canvas_attention (causal, long context)")
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    t = [to_dev(x, torch.bfloat16) for x in (q, kp, vp, kc, vc)]
    one = dg.dg_canvas_attention(*t, causal=True)
    bat = dg.dg_canvas_attention_batched(*[x[None] for x in t], [kp.shape[0]], [True])
    torch.cuda.synchronize()
    assert torch.equal(one, bat[0])
