"""Top-k truncated sampler steps on the device against the oracle (oracle.topk:
the untruncated oracle on logits with everything outside each row's kept set
at -inf).  Same comparison rules as the untruncated tests."""
import numpy as np
import pytest

import workloads
from gpu_util import check_step, check_z, log, require_gpu, to_dev
from oracle import sampler as S
from oracle import topk as K
from test_gpu_batch import canvas_ctrls, dev_ctrls
from test_gpu_eb import BUDGET, STOP, check_eb, spread_logits

pytestmark = pytest.mark.gpu


def tied_logits(rng, rows, vocab):
    """Noise rounded to 0.25 steps (many equal values, so the kept set is
    decided by ids at its edge), plus a spike in a third of the rows."""
    l = np.round(rng.standard_normal((rows, vocab)) * 8) / 4
    spikes = rng.random(rows) < 0.33
    l[np.nonzero(spikes)[0], rng.integers(0, vocab, spikes.sum())] += 9.0
    return l.astype(np.float32)


def run_topk(torch, dg, logits, emb, ids, mask, ctrls, k):
    rows = logits.shape[0]
    batch = len(ctrls)
    d = emb.shape[1]
    ids_t, mask_t = to_dev(ids.astype(np.int32)), to_dev(mask.astype(np.uint8))
    z = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    kappa = torch.empty(rows, dtype=torch.float32, device="cuda")
    nu = torch.zeros(batch, dtype=torch.int32, device="cuda")
    ctrl_t = dev_ctrls(dg, ctrls)
    dg.dg_sampler_step_topk(to_dev(logits), to_dev(emb), ids_t, mask_t, z, kappa, nu, ctrl_t, k, batch=batch)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (ids_t, mask_t, kappa, z, nu)] + [ctrl_t]


@pytest.mark.parametrize("n,batch,vocab,d,k", [
    (256, 1, 32768, 512, 64),
    (100, 3, 5003, 130, 17),       # unaligned vocabulary, ragged d, canvases sharing a pass
    (1, 5, 1000, 8, 256),
    (64, 2, 40000, 96, 1),         # five slices, the last one partial; k = 1
    (32, 1, 200, 64, 256),         # k >= vocab: the untruncated step
])
def test_topk_threshold_step(n, batch, vocab, d, k):
    torch, dg = require_gpu()
    log(f"top-k sampler n={n} batch={batch} V={vocab} d={d} k={k}")
    rng = np.random.default_rng(vocab + k)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    logits = tied_logits(rng, batch * n, vocab)
    ids = rng.integers(0, vocab, batch * n)
    mask = (rng.random(batch * n) < 0.2).astype(np.uint8)
    ctrls = canvas_ctrls(batch)
    g_ids, g_mask, g_kappa, g_z, g_nu, ctrl_t = run_topk(torch, dg, logits, emb, ids, mask, ctrls, k)
    e64 = emb.astype(np.float64)
    for b, c in enumerate(ctrls):
        sl = slice(b * n, (b + 1) * n)
        ref = K.sampler_step_topk(logits[sl], e64, ids[sl], mask[sl], c, k)
        assert check_step(ids[sl], mask[sl], g_ids[sl], g_mask[sl], g_kappa[sl], ref, c.tau) <= 1
        check_z(g_z[sl], ref["z"])
        assert g_nu[b] == n - int(g_mask[sl].sum())
        assert dg.read_ctrl(ctrl_t, b)["gstep"] == c.gstep + 1


def test_topk_kept_set_through_identity_embedding():
    """With E = I (V = d) z is the truncated distribution itself: its support is
    the kept set and its values the renormalised probabilities."""
    torch, dg = require_gpu()
    rng = np.random.default_rng(5)
    vocab, n = 512, 256
    logits = tied_logits(rng, n, vocab)
    logits[7] = 0.0                                   # all equal: the first k ids
    logits[8, :] = -np.inf
    logits[8, [3, 300, 511]] = [1.0, 1.0, 0.5]        # fewer finite logits than k
    emb = np.eye(vocab, dtype=np.float32)
    k = 37
    ctrl = S.Ctrl(seed=3, tau=2.0)
    _, _, _, g_z, _, _ = run_topk(torch, dg, logits, emb, np.zeros(n, int), np.zeros(n, np.uint8), [ctrl], k)
    for i in range(n):
        want = K.keep_mask(logits[i], k) & np.isfinite(logits[i])
        assert np.array_equal(g_z[i] > 0, want), f"row {i}: kept set differs"
    ref = K.sampler_step_topk(logits, emb.astype(np.float64), np.zeros(n, int), np.zeros(n, np.uint8), ctrl, k)
    check_z(g_z, ref["z"])
    np.testing.assert_allclose(g_z[7, :k], 1.0 / k, rtol=1e-6)


def test_topk_undefined_rows():
    torch, dg = require_gpu()
    rng = np.random.default_rng(8)
    n, vocab, d, k = 16, 20000, 32, 50
    logits = tied_logits(rng, n, vocab)
    logits[2, 19999] = np.nan
    logits[5, :] = -np.inf
    logits[9, 4] = np.inf
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    ids = rng.integers(0, vocab, n)
    ctrl = S.Ctrl(seed=2, tau=0.5)
    g_ids, g_mask, g_kappa, g_z, _, _ = run_topk(torch, dg, logits, emb, ids, np.zeros(n, np.uint8), [ctrl], k)
    ref = K.sampler_step_topk(logits, emb.astype(np.float64), ids, np.zeros(n, np.uint8), ctrl, k)
    check_step(ids, np.zeros(n, np.uint8), g_ids, g_mask, g_kappa, ref, ctrl.tau)
    assert np.isnan(g_kappa[[2, 5, 9]]).all() and not g_mask[[2, 5, 9]].any()
    assert np.isnan(g_z[[2, 5, 9]]).all()
    good = np.setdiff1d(np.arange(n), [2, 5, 9])
    check_z(g_z[good], ref["z"][good])


def test_topk_full_vocab_step():
    torch, dg = require_gpu()
    log("top-k full vocabulary: drawing inputs")
    emb = workloads.embedding(3)
    vocab, d = emb.shape
    n, k = 256, 64
    logits = workloads.step_logits(3, 0)
    ids = workloads.initial_canvas(3)[0].astype(np.int64)
    mask = np.zeros(n, np.uint8)
    ctrl = S.Ctrl(seed=11, gstep=1, flags=S.GUMBEL | S.AUTO_ADVANCE, tau=0.5, t_start=0.8, t_end=0.8)
    g_ids, g_mask, g_kappa, g_z, _, _ = run_topk(torch, dg, logits, emb, ids, mask, [ctrl], k)
    rows = np.array([0, 128, 255])
    log("  oracle")
    ref = K.sampler_step_topk(logits, emb.astype(np.float64), ids, mask, ctrl, k, z_rows=rows)
    assert check_step(ids, mask, g_ids, g_mask, g_kappa, ref, ctrl.tau) <= 1
    check_z(g_z[rows], ref["z"])
    log(f"  committed {int(g_mask.sum())} of {n}")


@pytest.mark.parametrize("n,batch,vocab,d,k", [(256, 1, 4096, 512, 32), (200, 2, 30000, 64, 100)])
def test_topk_entropy_bounded(n, batch, vocab, d, k):
    torch, dg = require_gpu()
    rng = np.random.default_rng(n + k)
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
    dg.dg_sampler_step_eb_topk(to_dev(logits), to_dev(emb), ids_t, acc, z, ent, amax, status, ctrl_t, k,
                               batch=batch, budget=BUDGET, stop_entropy=STOP)
    torch.cuda.synchronize()
    g = dict(ids=ids_t.cpu().numpy().astype(np.int64), accepted=acc.cpu().numpy(), entropy=ent.cpu().numpy(),
             argmax=amax.cpu().numpy().astype(np.int64), z=z.cpu().numpy())
    for b, c in enumerate(ctrls):
        sl = slice(b * n, (b + 1) * n)
        ref = K.eb_step_topk(logits[sl], emb, ids[sl], c, k, None, BUDGET, STOP, z_rows="all")
        got = {key: v[sl] for key, v in g.items()}
        got["status"] = dg.read_eb_status(status, b)
        assert check_eb(ref, got) <= 2
        check_z(got["z"], ref["z"])


def test_topk_degenerate_rows_take_the_overflow_paths():
    """Rows of equal logits put every candidate at the cut: more than 1024 keys
    reach a sub-slice's floor and more than 2048 the row's, so both fallback
    selects run; the kept set is then decided by ids alone."""
    torch, dg = require_gpu()
    rng = np.random.default_rng(12)
    n, vocab, d, k = 8, 40000, 32, 256
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[0] = 0.0                                        # all equal
    logits[1] = 1.5
    logits[1, rng.integers(0, vocab, 40)] = 3.0            # 40 at the top, the rest tied below
    logits[2, 20000:] = logits[2].max() + 1.0              # the upper half tied at the top
    logits[3] = -np.inf
    logits[3, [5, 39999]] = [0.0, -1.0]                    # two finite logits
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    ids = rng.integers(0, vocab, n)
    ctrl = S.Ctrl(seed=21, flags=S.GUMBEL, tau=0.05, t_start=0.9, t_end=0.9)
    g_ids, g_mask, g_kappa, g_z, _, _ = run_topk(torch, dg, logits, emb, ids, np.zeros(n, np.uint8), [ctrl], k)
    ref = K.sampler_step_topk(logits, emb.astype(np.float64), ids, np.zeros(n, np.uint8), ctrl, k)
    assert check_step(ids, np.zeros(n, np.uint8), g_ids, g_mask, g_kappa, ref, ctrl.tau) <= 1
    check_z(g_z, ref["z"])
    np.testing.assert_allclose(g_z[0], emb[:k].astype(np.float64).mean(0), rtol=1e-4, atol=1e-7)
