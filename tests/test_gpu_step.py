"""The whole denoising step (attention then sampler) eagerly and as a replayed HIP graph,
at the long-context, full-vocabulary shape, against the oracle."""
import numpy as np
import pytest

import workloads
from gpu_util import attention_reference, check_attention, check_step, check_z, log, require_gpu, to_dev
from oracle import sampler as S

pytestmark = pytest.mark.gpu

ROWS = np.array([0, 3, 64, 127, 128, 190, 255])


@pytest.fixture(scope="module")
def inputs():
    log("step: generating workload-4 inputs")
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    emb = workloads.embedding(3)
    logits = workloads.step_logits(4, 0)
    ids, mask = workloads.initial_canvas(4)
    attn_ref = attention_reference(q, kp, vp, kc, vc)
    return dict(q=q, kp=kp, vp=vp, kc=kc, vc=vc, emb=emb, logits=logits, ids=ids, mask=mask, attn_ref=attn_ref)


def device_state(torch, dg, x, ctrl):
    bf = torch.bfloat16
    st = dict(q=to_dev(x["q"], bf), kp=to_dev(x["kp"], bf), vp=to_dev(x["vp"], bf),
              kc=to_dev(x["kc"], bf), vc=to_dev(x["vc"], bf), emb=dg.dg_embedding_pack(to_dev(x["emb"])),
              logits=to_dev(x["logits"]), ids=to_dev(x["ids"].astype(np.int32)),
              mask=to_dev(x["mask"].astype(np.uint8)))
    n, hq, d = x["q"].shape
    st["attn"] = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    st["z"] = torch.empty((n, x["emb"].shape[1]), dtype=torch.float32, device="cuda")
    st["kappa"] = torch.empty(n, dtype=torch.float32, device="cuda")
    st["nu"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    st["ctrl"] = dg.make_ctrl(seed=ctrl.seed, gstep=ctrl.gstep, s_max=ctrl.s_max, flags=ctrl.flags,
                              tau=ctrl.tau, t_start=ctrl.t_start, t_end=ctrl.t_end)
    return st


def args(st):
    return (st["q"], st["kp"], st["vp"], st["kc"], st["vc"], st["attn"], st["logits"], st["emb"],
            st["ids"], st["mask"], st["z"], st["kappa"], st["nu"], st["ctrl"])


def snapshot(torch, st):
    torch.cuda.synchronize()
    return {k: st[k].cpu().numpy().copy() for k in ("attn", "ids", "mask", "kappa", "z", "nu", "ctrl")}


@pytest.mark.parametrize("flags", [S.AUTO_ADVANCE, S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE])
def test_eager_and_graph_steps(inputs, flags):
    torch, dg = require_gpu()
    ctrl = S.Ctrl(seed=4, tau=0.9, flags=flags, t_start=0.8, t_end=0.4)
    e64 = inputs["emb"].astype(np.float64)

    # eager: three steps on the same logits
    log("step: eager")
    st = device_state(torch, dg, inputs, ctrl)
    eager = []
    for _ in range(3):
        dg.dg_denoise_step(*args(st))
        eager.append(snapshot(torch, st))

    # the oracle, step by step
    ids, mask, c = inputs["ids"], inputs["mask"], ctrl
    for k in range(3):
        log(f"step: oracle step {k}")
        ref = S.sampler_step(inputs["logits"], e64, ids, mask, c, z_rows=ROWS)
        got = eager[k]
        check_attention(got["attn"], *inputs["attn_ref"], f"step {k} attention")
        assert check_step(ids, mask, got["ids"], got["mask"], got["kappa"], ref, 0.9) <= 2
        # both sides continue from the device's state (identical unless a decision fell in the band)
        ref = dict(ref, ids=got["ids"].astype(np.int64), committed=got["mask"])
        check_z(got["z"][ROWS], ref["z"])
        assert int(got["nu"][0]) == int(len(mask) - got["mask"].sum())
        ids, mask, c = ref["ids"], ref["committed"], ref["ctrl"]

    # graph: same three steps by replay, eager work and syncs in between
    log("step: graph")
    st = device_state(torch, dg, inputs, ctrl)
    graph = dg.StepGraph(*args(st))
    try:
        for k in range(3):
            graph.launch()
            got = snapshot(torch, st)
            scratch = torch.ones(1 << 20, device="cuda").sum().item()   # unrelated eager work
            assert scratch == float(1 << 20)
            for key in got:
                np.testing.assert_array_equal(got[key], eager[k][key], err_msg=f"replay {k} {key}")
            assert dg.read_ctrl(st["ctrl"])["gstep"] == k + 1
    finally:
        graph.close()


def test_entropy_bounded_step_eager_and_graph(inputs):
    """The step with the entropy-bounded sampler: eager steps against the oracle,
    then the same steps replayed from a captured graph, bit for bit."""
    from oracle import eb as EB
    from test_gpu_eb import BUDGET, STOP, check_eb
    torch, dg = require_gpu()
    flags = S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE
    ctrl = S.Ctrl(seed=8, s_max=48, flags=flags, t_start=0.8, t_end=0.4)
    n = inputs["q"].shape[0]

    def state():
        st = device_state(torch, dg, inputs, ctrl)
        st["ent"] = torch.empty(n, dtype=torch.float32, device="cuda")
        st["amax"] = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        st["status"] = torch.zeros(16, dtype=torch.uint8, device="cuda")
        return st

    def eb_args(st):
        return (st["q"], st["kp"], st["vp"], st["kc"], st["vc"], st["attn"], st["logits"], st["emb"], st["ids"],
                st["mask"], st["z"], st["ent"], st["amax"], st["status"], st["ctrl"])

    def snap(st):
        torch.cuda.synchronize()
        return {k: st[k].cpu().numpy().copy() for k in ("attn", "ids", "mask", "z", "ent", "amax", "status", "ctrl")}

    log("eb step: eager")
    st = state()
    eager = []
    for _ in range(3):
        dg.dg_denoise_step_eb(*eb_args(st), budget=BUDGET, stop_entropy=STOP)
        eager.append(snap(st))
    check_attention(eager[0]["attn"], *inputs["attn_ref"], "eb step attention")
    log("eb step: oracle step 0")
    ref = EB.eb_step(inputs["logits"], inputs["emb"].astype(np.float64), inputs["ids"], ctrl, None, BUDGET, STOP,
                     z_rows=ROWS)
    got = dict(ids=eager[0]["ids"].astype(np.int64), accepted=eager[0]["mask"], entropy=eager[0]["ent"],
               argmax=eager[0]["amax"].astype(np.int64), z=eager[0]["z"],
               status=dg.read_eb_status(torch.from_numpy(eager[0]["status"])))
    assert check_eb(ref, got) <= 2
    check_z(got["z"][ROWS], ref["z"])

    log("eb step: graph")
    st = state()
    graph = dg.StepGraphEB(*eb_args(st), budget=BUDGET, stop_entropy=STOP)
    try:
        for k in range(3):
            graph.launch()
            g = snap(st)
            assert torch.ones(1 << 20, device="cuda").sum().item() == float(1 << 20)   # unrelated eager work
            for key in g:
                np.testing.assert_array_equal(g[key], eager[k][key], err_msg=f"replay {k} {key}")
    finally:
        graph.close()


def test_fp8_step_eager_and_graph(inputs):
    """The step with FP8 attention inputs (scores on the FP8 matrix cores): the
    attention against the oracle on the decoded, scaled codes under the
    contract and the rounding bounds, the sampler against the oracle, then the
    same steps replayed from a captured graph, bit for bit."""
    from oracle import fp8 as F
    torch, dg = require_gpu()
    codes = workloads.attention_inputs_fp8(4)
    scales = (0.5, 0.75, 2.0)
    ctrl = S.Ctrl(seed=12, tau=0.9, flags=S.AUTO_ADVANCE)

    def state():
        st = device_state(torch, dg, inputs, ctrl)
        for k, c in zip(("q", "kp", "vp", "kc", "vc"), codes):
            st[k] = to_dev(c)
        return st

    def snap(st):
        torch.cuda.synchronize()
        return {k: st[k].cpu().numpy().copy() for k in ("attn", "ids", "mask", "kappa", "z", "nu", "ctrl")}

    log("fp8 step: eager")
    st = state()
    eager = []
    for _ in range(2):
        dg.dg_denoise_step_fp8(*args(st), *scales)
        eager.append(snap(st))
    qd, kpd, vpd, kcd, vcd = (F.e4m3_to_float(c) * float(np.float32(sc))
                              for c, sc in zip(codes, (scales[0], scales[1], scales[2], scales[1], scales[2])))
    ref_attn = attention_reference(qd, kpd, vpd, kcd, vcd)
    check_attention(eager[0]["attn"], ref_attn[0], ref_attn[1], ref_attn[2] * 1.0, "fp8 step attention")
    ref = S.sampler_step(inputs["logits"], inputs["emb"].astype(np.float64), inputs["ids"], inputs["mask"], ctrl,
                         z_rows=ROWS)
    assert check_step(inputs["ids"], inputs["mask"], eager[0]["ids"], eager[0]["mask"], eager[0]["kappa"], ref,
                      0.9) <= 2
    check_z(eager[0]["z"][ROWS], ref["z"])

    log("fp8 step: graph")
    st = state()
    graph = dg.StepGraphFP8(*args(st), *scales)
    try:
        for k in range(2):
            graph.launch()
            g = snap(st)
            assert torch.ones(1 << 20, device="cuda").sum().item() == float(1 << 20)   # unrelated eager work
            for key in g:
                np.testing.assert_array_equal(g[key], eager[k][key], err_msg=f"replay {k} {key}")
    finally:
        graph.close()
