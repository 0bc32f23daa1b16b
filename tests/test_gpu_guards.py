"""Guard words around every workspace and output buffer: each buffer is carved
from a larger allocation whose head and tail (4 KiB each) hold a NaN-payload
guard word, the entry point runs, and the guards must be unchanged afterwards.
A kernel writing past a workspace region's end or an output's end shows here
even when its results are right."""
import numpy as np
import pytest

import workloads
from gpu_util import log, require_gpu, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096                      # bytes before and after each buffer
WORD = 0x7FBADBAD                 # a NaN payload no kernel writes


class Guarded:
    """Device buffers carved from larger allocations with guard words around them."""

    def __init__(self, torch):
        self.torch = torch
        self.bufs = []

    def bytes(self, n):
        torch = self.torch
        words = (GUARD * 2 + ((int(n) + 255) // 256) * 256) // 4
        base = torch.full((words,), WORD, dtype=torch.int32, device="cuda")
        self.bufs.append((base, n))
        return base.view(torch.uint8)[GUARD:GUARD + int(n)]

    def tensor(self, shape, dtype):
        torch = self.torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return self.bytes(n).view(dtype).view(shape)

    def check(self, label):
        self.torch.cuda.synchronize()
        for base, n in self.bufs:
            b = base.cpu().numpy()
            head = b[:GUARD // 4]
            tail = b[(GUARD + ((int(n) + 3) // 4) * 4) // 4:]
            assert np.all(head == WORD), f"{label}: guard before a buffer of {n} bytes overwritten"
            assert np.all(tail == WORD), f"{label}: guard after a buffer of {n} bytes overwritten"


@pytest.mark.parametrize("n,p,hq,hkv,d,qkv,causal", [
    (256, 4096, 16, 8, 128, "bf16", False),
    (100, 37, 8, 2, 64, "f32", True),
    (64, 2048, 4, 2, 64, "bf16", False),
])
def test_attention_guards(n, p, hq, hkv, d, qkv, causal):
    torch, dg = require_gpu()
    log(f"guards: attention n={n} p={p} {qkv} causal={causal}")
    g = Guarded(torch)
    dt = torch.bfloat16 if qkv == "bf16" else torch.float32
    q, kp, vp, kc, vc = (to_dev(x, dt) for x in workloads.attention_inputs(2, n=n, n_prefix=p, hq=hq, hkv=hkv,
                                                                             head_dim=d, qkv=qkv))
    out = g.tensor((n, hq, d), torch.float32)
    ws = g.bytes(dg.dg_attention_workspace_bytes(n, p, hq, hkv, d))
    dg.dg_canvas_attention(q, kp, vp, kc, vc, out=out, workspace=ws, causal=causal)
    g.check("attention")
    assert torch.isfinite(out).all()


def test_fp8_and_batched_attention_guards():
    torch, dg = require_gpu()
    log("guards: fp8 and batched attention")
    g = Guarded(torch)
    n, p, hq, hkv, d = 256, 1024, 16, 8, 128
    codes = [to_dev(x) for x in workloads.attention_inputs_fp8(2, n=n, n_prefix=p)]
    out = g.tensor((n, hq, d), torch.float32)
    ws = g.bytes(dg.dg_attention_workspace_bytes(n, p, hq, hkv, d))
    dg.dg_canvas_attention_fp8(*codes, 0.5, 1.0, 2.0, out=out, workspace=ws)
    bf = torch.bfloat16
    q, kp, vp, kc, vc = (to_dev(x, bf) for x in workloads.attention_inputs(2, n=n, n_prefix=p))
    two = lambda x: torch.stack([x, x]).contiguous()
    outb = g.tensor((2, n, hq, d), torch.float32)
    wsb = g.bytes(dg.dg_attention_batched_workspace_bytes(2, n, p, hq, hkv, d))
    dg.dg_canvas_attention_batched(two(q), two(kp), two(vp), two(kc), two(vc), [p, 300], [False, True], out=outb,
                                   workspace=wsb)
    g.check("fp8 / batched attention")


@pytest.mark.parametrize("n,vocab,d,batch", [(256, 32768, 2048, 1), (17, 12345, 513, 3)])
def test_sampler_guards(n, vocab, d, batch):
    torch, dg = require_gpu()
    log(f"guards: sampler n={n} V={vocab} d={d} batch={batch}")
    g = Guarded(torch)
    rng = np.random.default_rng(5)
    rows = n * batch
    logits = to_dev((rng.standard_normal((rows, vocab)) * 3).astype(np.float32))
    emb = to_dev((rng.standard_normal((vocab, d)) * 0.02).astype(np.float32))
    packed = g.bytes(dg.dg_embedding_packed_bytes(vocab, d))
    dg.dg_embedding_pack(emb, packed=packed)
    ids = g.tensor((rows,), torch.int32)
    ids.copy_(torch.from_numpy(rng.integers(0, vocab, rows).astype(np.int32)))
    mask = g.tensor((rows,), torch.uint8)
    mask.zero_()
    z = g.tensor((rows, d), torch.float32)
    kappa = g.tensor((rows,), torch.float32)
    nu = g.tensor((batch,), torch.int32)
    ctrl = dg.stack_ctrl([dg.make_ctrl(seed=3 + b, tau=0.9, flags=dg.DG_AUTO_ADVANCE) for b in range(batch)])
    ws = g.bytes(dg.dg_sampler_workspace_bytes_batched(n, batch, vocab, d))
    dg.dg_sampler_step_batched(logits, packed, ids, mask, z, kappa, nu, ctrl, batch, workspace=ws)
    g.check("sampler")
    # entropy-bounded mode on the same buffers
    ent = g.tensor((rows,), torch.float32)
    amax = g.tensor((rows,), torch.int32)
    amax.fill_(-1)
    status = g.tensor((16 * batch,), torch.uint8)
    dg.dg_sampler_step_eb_batched(logits, packed, ids, mask, z, ent, amax, status, ctrl, batch, workspace=ws)
    g.check("entropy-bounded sampler")
    # top-k mode (its own workspace)
    wst = g.bytes(dg.dg_sampler_workspace_bytes_topk(n, batch, vocab, d, 64))
    dg.dg_sampler_step_topk(logits, emb, ids, mask, z, kappa, nu, ctrl, 64, batch=batch, workspace=wst)
    g.check("top-k sampler")


def test_denoise_step_guards():
    """The whole long-context step, eagerly and as a graph replay, with every
    buffer it writes (and its one shared workspace) guarded."""
    torch, dg = require_gpu()
    log("guards: denoising step at the long-context, full-vocabulary shape")
    g = Guarded(torch)
    c = workloads.CONFIGS[4]
    n, p, hq, hkv, d, vocab, dm = c["n"], c["n_prefix"], c["hq"], c["hkv"], c["head_dim"], c["vocab"], c["d_model"]
    bf = torch.bfloat16
    q, kp, vp, kc, vc = (to_dev(x, bf) for x in workloads.attention_inputs(4))
    logits = to_dev(workloads.step_logits(4, 0))
    emb = to_dev(workloads.embedding(4))
    packed = g.bytes(dg.dg_embedding_packed_bytes(vocab, dm))
    dg.dg_embedding_pack(emb, packed=packed)
    del emb
    ids0, _ = workloads.initial_canvas(4)
    ids = g.tensor((n,), torch.int32)
    ids.copy_(torch.from_numpy(ids0.astype(np.int32)))
    mask = g.tensor((n,), torch.uint8)
    mask.zero_()
    attn = g.tensor((n, hq, d), torch.float32)
    z = g.tensor((n, dm), torch.float32)
    kappa = g.tensor((n,), torch.float32)
    nu = g.tensor((1,), torch.int32)
    ctrl = dg.make_ctrl(seed=4, tau=0.9, flags=dg.DG_AUTO_ADVANCE)
    ws = g.bytes(dg.dg_denoise_workspace_bytes(n, p, hq, hkv, d, vocab, dm))
    args = (q, kp, vp, kc, vc, attn, logits, packed, ids, mask, z, kappa, nu, ctrl)
    dg.dg_denoise_step(*args, workspace=ws)
    g.check("denoise step")
    graph = dg.StepGraph(*args, workspace=ws)
    try:
        graph.launch()
        graph.launch()
    finally:
        graph.close()
    g.check("denoise step graph")
