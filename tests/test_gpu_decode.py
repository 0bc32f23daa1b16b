"""The decode run: a 4096-token prefix, then four 256-token canvases, each denoised
until committed with Gumbel candidates and the linear temperature schedule, the
logits drawn on the device by the threshold-tuned synthetic generator, and each
finished canvas appended to the KV cache before the next one starts.

Each canvas runs through one captured step graph (canvas attention over the
prefix as it stands, then the sampler; the prefix grows by 256 rows per canvas)
replayed once per step, with the synthetic logits written before each replay.
Every step is compared with the oracle from the same entry state: the device's
synthetic logits bit for bit, the attention output (against the oracle on the
first step of a canvas, bit-identical on the later replays), ids / commit mask /
confidence under the comparison rules, z on sampled rows, the counter of open
positions and the control block.  Each test runs one canvas; they share the
run's state and go in order.
"""
import numpy as np
import pytest

import workloads
from gpu_util import attention_reference, check_attention, check_step, check_z, log, require_gpu, to_dev
from oracle import sampler as S
from oracle import synth

pytestmark = pytest.mark.gpu

CFG = workloads.CONFIGS[5]
ROWS = np.array([0, 17, 128, 255])
FLAGS = S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE


@pytest.fixture(scope="module")
def run():
    torch, dg = require_gpu()
    n, p0, hkv, hd, vocab = CFG["n"], CFG["n_prefix"], CFG["hkv"], CFG["head_dim"], CFG["vocab"]
    log("decode: drawing E and the prefix")
    emb = workloads.embedding(5)
    q, kp, vp, _, _ = workloads.attention_inputs(5, block=0)
    table = workloads.synth_table()
    bf = torch.bfloat16
    total = p0 + CFG["blocks"] * n
    kbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    vbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    kbuf[:p0] = to_dev(kp, bf)
    vbuf[:p0] = to_dev(vp, bf)
    ctrl = S.Ctrl(seed=CFG["seed"], s_max=CFG["s_max"], flags=FLAGS, tau=CFG["tau"],
                  t_start=CFG["t_start"], t_end=CFG["t_end"])
    st = dict(
        emb=dg.dg_embedding_pack(to_dev(emb)), table=to_dev(table),
        kbuf=kbuf, vbuf=vbuf, n_prefix=p0,
        logits=torch.empty((n, vocab), dtype=torch.float32, device="cuda"),
        ids=torch.zeros(n, dtype=torch.int32, device="cuda"),
        mask=torch.zeros(n, dtype=torch.uint8, device="cuda"),
        z=torch.empty((n, emb.shape[1]), dtype=torch.float32, device="cuda"),
        kappa=torch.empty(n, dtype=torch.float32, device="cuda"),
        nu=torch.zeros(1, dtype=torch.int32, device="cuda"),
        ctrl=dg.make_ctrl(seed=ctrl.seed, s_max=ctrl.s_max, flags=ctrl.flags, tau=ctrl.tau,
                          t_start=ctrl.t_start, t_end=ctrl.t_end),
        attn=torch.empty((n, CFG["hq"], hd), dtype=torch.float32, device="cuda"),
        # one workspace for every canvas's step graph: sized for the longest prefix
        ws=torch.empty(dg.dg_denoise_workspace_bytes(n, total - n, CFG["hq"], hkv, hd, vocab, emb.shape[1]),
                       dtype=torch.uint8, device="cuda"),
        # oracle side
        e64=emb.astype(np.float64), table_np=table, kp=kp, vp=vp, ctrl_ref=ctrl,
        steps=[], torch=torch, dg=dg)
    del emb
    yield st


def ctrl_matches(dg, ctrl_t, c):
    got = dg.read_ctrl(ctrl_t)
    return got["gstep"] == c.gstep and got["s_in_block"] == c.s_in_block


@pytest.mark.timeout(600)
@pytest.mark.parametrize("block", range(CFG["blocks"]))
def test_decode_block(run, block):
    torch, dg = run["torch"], run["dg"]
    n, vocab, hq, hkv, hd = CFG["n"], CFG["vocab"], CFG["hq"], CFG["hkv"], CFG["head_dim"]
    assert len(run["steps"]) == block, "blocks run in order"
    bf = torch.bfloat16
    q, _, _, kc, vc = workloads.attention_inputs(5, block=block)
    p = run["n_prefix"]

    kp_d, vp_d = run["kbuf"][:p], run["vbuf"][:p]
    q_d, kc_d, vc_d = to_dev(q, bf), to_dev(kc, bf), to_dev(vc, bf)
    attn_ref = attention_reference(q, run["kp"], run["vp"], kc, vc)

    # a fresh canvas
    dg.dg_canvas_init(run["ids"], run["mask"], run["ctrl"], vocab)
    ids, mask, c = S.init_canvas(run["ctrl_ref"], n, vocab)
    torch.cuda.synchronize()
    assert np.array_equal(run["ids"].cpu().numpy(), ids)
    assert not run["mask"].cpu().numpy().any()
    assert ctrl_matches(dg, run["ctrl"], c)

    # this canvas's step graph: attention over the prefix of p rows, then the sampler
    graph = dg.StepGraph(q_d, kp_d, vp_d, kc_d, vc_d, run["attn"], run["logits"], run["emb"], run["ids"],
                         run["mask"], run["z"], run["kappa"], run["nu"], run["ctrl"], workspace=run["ws"])
    accepted = []
    attn0 = None
    try:
        while True:
            dg.dg_synth_logits(run["logits"], run["ids"], run["mask"], run["ctrl"], run["table"])
            torch.cuda.synchronize()
            logits = synth.synth_logits(ids, mask, c.gstep, c.seed, run["table_np"], vocab)
            assert np.array_equal(run["logits"].cpu().numpy(), logits), "synthetic logits differ"
            graph.launch()
            torch.cuda.synchronize()
            attn = run["attn"].cpu().numpy()
            if attn0 is None:
                check_attention(attn, *attn_ref, f"decode block {block} (prefix {p}) attention")
                attn0 = attn
            else:
                assert np.array_equal(attn, attn0), "attention differs between replays"
            ref = S.sampler_step(logits, run["e64"], ids, mask, c, z_rows=ROWS)
            g_ids, g_mask = run["ids"].cpu().numpy(), run["mask"].cpu().numpy()
            exempt = check_step(ids, mask, g_ids, g_mask, run["kappa"].cpu().numpy(), ref, c.tau)
            check_z(run["z"].cpu().numpy()[ROWS], ref["z"])
            assert int(run["nu"].cpu()[0]) == int(n - g_mask.sum())
            c = ref["ctrl"]
            assert ctrl_matches(dg, run["ctrl"], c)
            accepted.append(int(g_mask.sum() - mask.sum()))
            # both sides continue from the device's state (identical unless a decision
            # fell inside the comparison band)
            ids, mask = g_ids.astype(np.int64), g_mask
            if exempt:
                log(f"decode block {block}: step {len(accepted)}: {exempt} in-band decisions")
            if int(run["nu"].cpu()[0]) == 0:
                break
            assert len(accepted) < CFG["s_max"], "canvas did not finish within the step budget"
    finally:
        graph.close()
    run["ctrl_ref"] = c
    log(f"decode block {block}: {len(accepted)} steps, accepted per step {accepted}")
    # about 20 tokens per forward pass, as the generator is tuned for
    assert 10 <= len(accepted) <= 20
    assert 15.0 <= n / len(accepted) <= 26.0

    # the finished canvas joins the KV cache
    dg.dg_kv_append(run["kbuf"], run["vbuf"], kc_d, vc_d, p)
    run["kp"] = np.concatenate([run["kp"], kc], axis=0)
    run["vp"] = np.concatenate([run["vp"], vc], axis=0)
    run["n_prefix"] = p + n
    torch.cuda.synchronize()
    got_k = run["kbuf"][:p + n].float().cpu().numpy()
    got_v = run["vbuf"][:p + n].float().cpu().numpy()
    assert np.array_equal(got_k, run["kp"]) and np.array_equal(got_v, run["vp"])
    run["steps"].append(accepted)
    if block == CFG["blocks"] - 1:
        total = sum(sum(a) for a in run["steps"])
        n_steps = sum(len(a) for a in run["steps"])
        log(f"decode: {total} tokens in {n_steps} steps ({total / n_steps:.1f} per step)")
        assert total == CFG["blocks"] * n
