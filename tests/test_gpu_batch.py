"""A batch of canvases in one sampler pass: every canvas must match the oracle
run on that canvas alone (its own control block, seed, step and flags), under
the same comparison rules as the single-canvas tests."""
import numpy as np
import pytest

import workloads
from gpu_util import check_step, check_z, log, require_gpu, to_dev
from oracle import eb as EB
from oracle import sampler as S
from test_gpu_eb import BUDGET, STOP, check_eb, spread_logits

pytestmark = pytest.mark.gpu


def canvas_ctrls(batch):
    """Different seeds, steps, flags and temperatures per canvas."""
    out = []
    for b in range(batch):
        flags = S.AUTO_ADVANCE | (S.GUMBEL if b % 2 else 0) | (S.T_SCHEDULE if b % 3 == 2 else 0)
        out.append(S.Ctrl(seed=100 + 7 * b, gstep=3 * b, s_in_block=b, s_max=48, flags=flags, tau=0.9,
                          t_start=0.8 if flags & S.T_SCHEDULE else 1.0, t_end=0.4 if flags & S.T_SCHEDULE else 1.0))
    return out


def dev_ctrls(dg, ctrls):
    return dg.stack_ctrl([dg.make_ctrl(seed=c.seed, gstep=c.gstep, s_in_block=c.s_in_block, s_max=c.s_max,
                                       flags=c.flags, tau=c.tau, t_start=c.t_start, t_end=c.t_end)
                          for c in ctrls])


@pytest.mark.parametrize("n,batch,vocab,d", [
    (256, 3, 32768, 512),
    (100, 5, 5003, 130),     # ragged canvases: a 256-row tile spans canvases
    (1, 7, 2048, 64),
])
def test_batched_threshold_step(n, batch, vocab, d):
    torch, dg = require_gpu()
    log(f"batched sampler n={n} batch={batch} V={vocab} d={d}")
    rng = np.random.default_rng(n + 13 * batch)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    logits = (rng.standard_normal((batch * n, vocab)) * 3).astype(np.float32)
    spikes = rng.random(batch * n) < 0.3
    logits[np.nonzero(spikes)[0], rng.integers(0, vocab, spikes.sum())] += 14.0
    ids = rng.integers(0, vocab, batch * n).astype(np.int32)
    mask = (rng.random(batch * n) < 0.2).astype(np.uint8)
    ctrls = canvas_ctrls(batch)
    ids_t, mask_t = to_dev(ids), to_dev(mask)
    z = torch.empty((batch * n, d), dtype=torch.float32, device="cuda")
    kappa = torch.empty(batch * n, dtype=torch.float32, device="cuda")
    nu = torch.zeros(batch, dtype=torch.int32, device="cuda")
    ctrl_t = dev_ctrls(dg, ctrls)
    dg.dg_sampler_step_batched(to_dev(logits), dg.dg_embedding_pack(to_dev(emb)), ids_t, mask_t, z, kappa,
                               nu, ctrl_t, batch)
    torch.cuda.synchronize()
    g_ids, g_mask, g_kappa, g_z, g_nu = (x.cpu().numpy() for x in (ids_t, mask_t, kappa, z, nu))
    e64 = emb.astype(np.float64)
    for b, c in enumerate(ctrls):
        sl = slice(b * n, (b + 1) * n)
        rows = np.unique(np.array([0, n // 2, n - 1]))
        ref = S.sampler_step(logits[sl], e64, ids[sl], mask[sl], c, z_rows=rows)
        assert check_step(ids[sl], mask[sl], g_ids[sl], g_mask[sl], g_kappa[sl], ref, c.tau) <= 1
        check_z(g_z[sl][rows], ref["z"])
        assert g_nu[b] == n - int(g_mask[sl].sum())
        got_c = dg.read_ctrl(ctrl_t, b)
        assert got_c["gstep"] == c.gstep + 1 and got_c["s_in_block"] == c.s_in_block + 1


def test_batched_full_vocab():
    """Four canvases of the full-vocabulary shape share one pass over E."""
    torch, dg = require_gpu()
    batch, n = 4, 256
    log("batched full vocabulary: drawing inputs")
    emb = workloads.embedding(3)
    vocab, d = emb.shape
    logits = np.concatenate([workloads.step_logits(3, b) for b in range(batch)])
    ids = np.concatenate([workloads.initial_canvas(3)[0] for _ in range(batch)]).astype(np.int32)
    mask = np.zeros(batch * n, np.uint8)
    ctrls = canvas_ctrls(batch)
    ids_t, mask_t = to_dev(ids), to_dev(mask)
    z = torch.empty((batch * n, d), dtype=torch.float32, device="cuda")
    kappa = torch.empty(batch * n, dtype=torch.float32, device="cuda")
    nu = torch.zeros(batch, dtype=torch.int32, device="cuda")
    ctrl_t = dev_ctrls(dg, ctrls)
    dg.dg_sampler_step_batched(to_dev(logits), dg.dg_embedding_pack(to_dev(emb)), ids_t, mask_t, z, kappa,
                               nu, ctrl_t, batch)
    torch.cuda.synchronize()
    g_ids, g_mask, g_kappa, g_z = (x.cpu().numpy() for x in (ids_t, mask_t, kappa, z))
    e64 = emb.astype(np.float64)
    rows = np.array([0, 97, 255])
    for b, c in enumerate(ctrls):
        log(f"  canvas {b}: oracle")
        sl = slice(b * n, (b + 1) * n)
        ref = S.sampler_step(logits[sl], e64, ids[sl], mask[sl], c, z_rows=rows)
        assert check_step(ids[sl], mask[sl], g_ids[sl], g_mask[sl], g_kappa[sl], ref, c.tau) <= 1
        check_z(g_z[sl][rows], ref["z"])


def test_batched_entropy_bounded():
    torch, dg = require_gpu()
    batch, n, vocab, d = 3, 200, 4096, 96
    rng = np.random.default_rng(77)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    logits = spread_logits(rng, batch * n, vocab)
    ids = rng.integers(0, vocab, batch * n)
    ctrls = canvas_ctrls(batch)
    ids_t = to_dev(ids.astype(np.int32))
    acc = torch.zeros(batch * n, dtype=torch.uint8, device="cuda")
    z = torch.empty((batch * n, d), dtype=torch.float32, device="cuda")
    ent = torch.empty(batch * n, dtype=torch.float32, device="cuda")
    amax = torch.full((batch * n,), -1, dtype=torch.int32, device="cuda")
    status = torch.zeros(16 * batch, dtype=torch.uint8, device="cuda")
    ctrl_t = dev_ctrls(dg, ctrls)
    dg.dg_sampler_step_eb_batched(to_dev(logits), dg.dg_embedding_pack(to_dev(emb)), ids_t, acc, z, ent, amax,
                                  status, ctrl_t, batch, BUDGET, STOP)
    torch.cuda.synchronize()
    g = dict(ids=ids_t.cpu().numpy().astype(np.int64), accepted=acc.cpu().numpy(), entropy=ent.cpu().numpy(),
             argmax=amax.cpu().numpy().astype(np.int64), z=z.cpu().numpy())
    for b, c in enumerate(ctrls):
        sl = slice(b * n, (b + 1) * n)
        ref = EB.eb_step(logits[sl], emb, ids[sl], c, None, BUDGET, STOP, z_rows=None)
        got = {k: v[sl] for k, v in g.items()}
        got["status"] = dg.read_eb_status(status, b)
        check_eb(ref, got)
