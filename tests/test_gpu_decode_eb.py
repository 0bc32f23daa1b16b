"""A decode run in the pages' default mode: each canvas is denoised by the
entropy-bounded sampler until adaptive stopping fires (explainer "DiffusionGemma:
Google's open diffusion LLM", sections "A diffusion language model refines 256
tokens in 12 steps" and Table 2), with Gumbel candidates and the linear
temperature schedule.  The logits come from the device's synthetic generator,
with the accepted positions in the place of the committed mask, so an accepted
position keeps its spike at its own id and about 20 new positions spike per
step.

Every step is compared with the oracle from the device's entry state: the
synthetic logits bit for bit, then entropies, acceptance, ids, the stop flag and
z on sampled rows under the entropy-bounded comparison rules.
"""
import numpy as np
import pytest

import workloads
from gpu_util import check_z, log, require_gpu, to_dev
from oracle import eb as EB
from oracle import sampler as S
from oracle import synth
from test_gpu_eb import BUDGET, STOP, check_eb

pytestmark = pytest.mark.gpu

ROWS = np.array([0, 99, 255])


def test_entropy_bounded_decode_run():
    torch, dg = require_gpu()
    n, vocab, d, s_max, canvases = 256, 32768, 256, 48, 2
    rng = np.random.default_rng(2024)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    table = workloads.synth_table()
    flags = S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE
    ctrl = S.Ctrl(seed=515, s_max=s_max, flags=flags, tau=0.9, t_start=0.8, t_end=0.4)
    d_ctrl = dg.make_ctrl(seed=ctrl.seed, s_max=s_max, flags=flags, tau=ctrl.tau, t_start=0.8, t_end=0.4)
    packed = dg.dg_embedding_pack(to_dev(emb))
    table_t = to_dev(table)
    logits = torch.empty((n, vocab), dtype=torch.float32, device="cuda")
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    acc = torch.zeros(n, dtype=torch.uint8, device="cuda")
    z = torch.empty((n, d), dtype=torch.float32, device="cuda")
    ent = torch.empty(n, dtype=torch.float32, device="cuda")
    amax = torch.empty(n, dtype=torch.int32, device="cuda")
    status = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.empty(dg.dg_sampler_workspace_bytes(n, vocab, d), dtype=torch.uint8, device="cuda")
    for c in range(canvases):
        dg.dg_canvas_init(ids, acc, d_ctrl, vocab)
        amax.fill_(-1)
        torch.cuda.synchronize()
        ref_ids, _, ctrl = S.init_canvas(ctrl, n, vocab)
        assert np.array_equal(ids.cpu().numpy(), ref_ids), "canvas initialisation differs"
        accepted = np.zeros(n, np.uint8)
        prev = None
        counts = []
        for step in range(s_max):
            dg.dg_synth_logits(logits, ids, acc, d_ctrl, table_t)
            dev_ids = ids.cpu().numpy().astype(np.int64)
            dev_acc = acc.cpu().numpy()
            ref_logits = synth.synth_logits(dev_ids, dev_acc, ctrl.gstep, ctrl.seed, table, vocab)
            assert np.array_equal(logits.cpu().numpy(), ref_logits), f"canvas {c} step {step}: logits differ"
            dg.dg_sampler_step_eb(logits, packed, ids, acc, z, ent, amax, status, d_ctrl, BUDGET, STOP,
                                  workspace=ws)
            torch.cuda.synchronize()
            got = dict(ids=ids.cpu().numpy().astype(np.int64), accepted=acc.cpu().numpy(),
                       entropy=ent.cpu().numpy(), argmax=amax.cpu().numpy().astype(np.int64),
                       z=z.cpu().numpy(), status=dg.read_eb_status(status))
            ref = EB.eb_step(ref_logits, emb.astype(np.float64), dev_ids, ctrl, prev, BUDGET, STOP, z_rows=ROWS)
            check_eb(ref, got)
            check_z(got["z"][ROWS], ref["z"])
            counts.append(int(got["status"]["n_accepted"]))
            prev, ctrl = got["argmax"], ref["ctrl"]
            if got["status"]["stop"]:
                break
        log(f"canvas {c}: stopped after {step + 1} steps, accepted per step {counts}")
        assert got["status"]["stop"] and step + 1 < s_max
        assert np.array_equal(got["ids"], got["argmax"])
        assert max(counts) == n and counts[0] >= 10


@pytest.mark.timeout(900)
def test_entropy_bounded_decode_run_through_step_graphs():
    """The decode-run shapes in the pages' default mode, each canvas through one
    captured step graph (canvas attention over the prefix as it stands, then the
    entropy-bounded sampler; the prefix grows by 256 rows per canvas).  Two
    canvases over a 4096-token prefix, 262144 ids, d_model 3072: per step the
    synthetic logits bit for bit, the attention against the oracle on the first
    step of a canvas and bit-identical on the later replays, and the sampler
    against the oracle from the device's entry state."""
    from gpu_util import attention_reference, check_attention
    torch, dg = require_gpu()
    cfg = workloads.CONFIGS[5]
    n, p0, hq, hkv, hd, vocab = cfg["n"], cfg["n_prefix"], cfg["hq"], cfg["hkv"], cfg["head_dim"], cfg["vocab"]
    canvases, s_max = 2, cfg["s_max"]
    log("eb decode (graphs): drawing E and the prefix")
    emb = workloads.embedding(5)
    d = emb.shape[1]
    _, kp, vp, _, _ = workloads.attention_inputs(5, block=0)
    table = workloads.synth_table()
    bf = torch.bfloat16
    total = p0 + canvases * n
    kbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    vbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    kbuf[:p0] = to_dev(kp, bf)
    vbuf[:p0] = to_dev(vp, bf)
    flags = S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE
    ctrl = S.Ctrl(seed=cfg["seed"], s_max=s_max, flags=flags, tau=cfg["tau"], t_start=cfg["t_start"],
                  t_end=cfg["t_end"])
    d_ctrl = dg.make_ctrl(seed=ctrl.seed, s_max=s_max, flags=flags, tau=ctrl.tau, t_start=ctrl.t_start,
                          t_end=ctrl.t_end)
    packed = dg.dg_embedding_pack(to_dev(emb))
    e64 = emb.astype(np.float64)
    del emb
    table_t = to_dev(table)
    logits = torch.empty((n, vocab), dtype=torch.float32, device="cuda")
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    acc = torch.zeros(n, dtype=torch.uint8, device="cuda")
    z = torch.empty((n, d), dtype=torch.float32, device="cuda")
    ent = torch.empty(n, dtype=torch.float32, device="cuda")
    amax = torch.empty(n, dtype=torch.int32, device="cuda")
    status = torch.zeros(16, dtype=torch.uint8, device="cuda")
    attn = torch.empty((n, hq, hd), dtype=torch.float32, device="cuda")
    ws = torch.empty(dg.dg_denoise_workspace_bytes(n, total - n, hq, hkv, hd, vocab, d), dtype=torch.uint8,
                     device="cuda")
    kp_all, vp_all = kp, vp
    p = p0
    for c in range(canvases):
        q, _, _, kc, vc = workloads.attention_inputs(5, block=c)
        q_d, kc_d, vc_d = to_dev(q, bf), to_dev(kc, bf), to_dev(vc, bf)
        attn_ref = attention_reference(q, kp_all, vp_all, kc, vc)
        dg.dg_canvas_init(ids, acc, d_ctrl, vocab)
        amax.fill_(-1)
        torch.cuda.synchronize()
        ref_ids, _, ctrl = S.init_canvas(ctrl, n, vocab)
        assert np.array_equal(ids.cpu().numpy(), ref_ids), "canvas initialisation differs"
        graph = dg.StepGraphEB(q_d, kbuf[:p], vbuf[:p], kc_d, vc_d, attn, logits, packed, ids, acc, z, ent, amax,
                               status, d_ctrl, budget=BUDGET, stop_entropy=STOP, workspace=ws)
        prev, counts, attn0 = None, [], None
        try:
            for step in range(s_max):
                dg.dg_synth_logits(logits, ids, acc, d_ctrl, table_t)
                dev_ids = ids.cpu().numpy().astype(np.int64)
                dev_acc = acc.cpu().numpy()
                ref_logits = synth.synth_logits(dev_ids, dev_acc, ctrl.gstep, ctrl.seed, table, vocab)
                assert np.array_equal(logits.cpu().numpy(), ref_logits), f"canvas {c} step {step}: logits differ"
                graph.launch()
                torch.cuda.synchronize()
                a = attn.cpu().numpy()
                if attn0 is None:
                    check_attention(a, *attn_ref, f"eb decode canvas {c} (prefix {p}) attention")
                    attn0 = a
                else:
                    assert np.array_equal(a, attn0), "attention differs between replays"
                got = dict(ids=ids.cpu().numpy().astype(np.int64), accepted=acc.cpu().numpy(),
                           entropy=ent.cpu().numpy(), argmax=amax.cpu().numpy().astype(np.int64),
                           z=z.cpu().numpy(), status=dg.read_eb_status(status))
                ref = EB.eb_step(ref_logits, e64, dev_ids, ctrl, prev, BUDGET, STOP, z_rows=ROWS)
                check_eb(ref, got)
                check_z(got["z"][ROWS], ref["z"])
                counts.append(int(got["status"]["n_accepted"]))
                prev, ctrl = got["argmax"], ref["ctrl"]
                if got["status"]["stop"]:
                    break
        finally:
            graph.close()
        log(f"eb decode (graphs) canvas {c}: stopped after {step + 1} steps, accepted per step {counts}")
        assert got["status"]["stop"] and step + 1 < s_max
        dg.dg_kv_append(kbuf, vbuf, kc_d, vc_d, p)
        kp_all = np.concatenate([kp_all, kc], axis=0)
        vp_all = np.concatenate([vp_all, vc], axis=0)
        p += n
