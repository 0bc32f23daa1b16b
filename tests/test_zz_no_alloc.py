"""The no-allocation attention entry point (dg_canvas_attention_noalloc) on the
GPU: its output equals dg_canvas_attention_ex's bit for bit on the same inputs
(same kernels, same plan, the static scratch in place of the workspace), on two
calls in a row, the second smaller than the first, and both meet the oracle's
bounds."""
import numpy as np
import pytest

import workloads
from gpu_util import attention_reference, check_attention, log, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def test_noalloc_matches_the_workspace_entry_point():
    torch, dg = require_gpu()
    cases = [
        # (workload recipe overrides, dtype, causal): the long-context shape, then a smaller ragged one
        (dict(), "bf16", False),
        (dict(n=100, n_prefix=37, hq=8, hkv=2, head_dim=64, qkv="f32"), "f32", True),
    ]
    for k, (over, qkv, causal) in enumerate(cases):
        log(f"noalloc call {k}: {over or 'long-context shape'} {qkv} causal={causal}")
        q, kp, vp, kc, vc = workloads.attention_inputs(4 if not over else 2, **over)
        dt = torch.bfloat16 if qkv == "bf16" else torch.float32
        t = [to_dev(x, dt) for x in (q, kp, vp, kc, vc)]
        n, hq, d = q.shape
        out_ws = dg.dg_canvas_attention(*t, causal=causal)
        out_na = torch.full((n, hq, d), float("nan"), dtype=torch.float32, device="cuda")
        dg.dg_canvas_attention_noalloc(*t, out_na, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out_ws, out_na), f"call {k}: noalloc output differs from the workspace entry point"
        ref, ref_r, bound = attention_reference(q, kp, vp, kc, vc, causal=causal, staged_bf16=(qkv == "f32"))
        check_attention(out_na.cpu().numpy(), ref, ref_r, bound, f"noalloc call {k}")
