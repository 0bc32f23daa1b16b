"""Entropy-bounded sampler steps and adaptive stopping on the device, against the oracle.

Comparison rules (the entropy-bounded analogue of the threshold rules):
  - entropies agree within 1e-5 + 1e-5 * H (fp32 sums over the vocabulary vs fp64);
  - greedy argmax ids are identical;
  - a position's acceptance may differ only if the oracle's running sum at its
    rank is within 1e-4 of the budget, or its entropy is within 2e-5 of another
    row's (order ambiguity);
  - where both sides accept, ids equal the oracle's candidate unless its top-2
    gap is within 1e-4; where neither accepts, ids equal the re-noise draw exactly;
  - the stop flag agrees unless the mean entropy is within 1e-5 of the threshold;
    when both stop, ids are the greedy argmax ids.
"""
import numpy as np
import pytest

import workloads
from gpu_util import BAND, check_z, log, require_gpu, to_dev
from oracle import eb as EB
from oracle import sampler as S

pytestmark = pytest.mark.gpu

BUDGET = float(np.float32(EB.BUDGET))
STOP = float(np.float32(EB.STOP_ENTROPY))


class DevEb:
    """Device buffers for one canvas in entropy-bounded mode."""

    def __init__(self, torch, dg, emb, n, ctrl):
        self.torch, self.dg = torch, dg
        vocab, d = emb.shape
        self.vocab, self.d, self.n = vocab, d, n
        self.emb = dg.dg_embedding_pack(to_dev(emb))
        self.ids = torch.zeros(n, dtype=torch.int32, device="cuda")
        self.acc = torch.zeros(n, dtype=torch.uint8, device="cuda")
        self.z = torch.empty((n, d), dtype=torch.float32, device="cuda")
        self.ent = torch.empty(n, dtype=torch.float32, device="cuda")
        self.argmax = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        self.status = torch.zeros(16, dtype=torch.uint8, device="cuda")
        self.ctrl = dg.make_ctrl(seed=ctrl.seed, gstep=ctrl.gstep, s_in_block=ctrl.s_in_block,
                                 s_max=ctrl.s_max, flags=ctrl.flags, tau=ctrl.tau,
                                 t_start=ctrl.t_start, t_end=ctrl.t_end)
        self.ws = torch.empty(dg.dg_sampler_workspace_bytes(n, vocab, d), dtype=torch.uint8, device="cuda")

    def step(self, logits_t, ids_np=None):
        if ids_np is not None:
            self.ids.copy_(to_dev(np.asarray(ids_np, np.int32)))
        self.dg.dg_sampler_step_eb(logits_t, self.emb, self.ids, self.acc, self.z, self.ent, self.argmax,
                                   self.status, self.ctrl, BUDGET, STOP, workspace=self.ws)
        self.torch.cuda.synchronize()
        return dict(ids=self.ids.cpu().numpy().astype(np.int64), accepted=self.acc.cpu().numpy(),
                    entropy=self.ent.cpu().numpy(), argmax=self.argmax.cpu().numpy().astype(np.int64),
                    z=self.z.cpu().numpy(), status=self.dg.read_eb_status(self.status),
                    ctrl=self.dg.read_ctrl(self.ctrl))


def check_eb(ref, got):
    """Apply the comparison rules; returns the number of exempt positions."""
    h = ref["entropy"]
    fin = ~np.isnan(h)
    assert np.array_equal(np.isnan(got["entropy"]), ~fin), "undefined rows differ"
    err = np.abs(got["entropy"][fin].astype(np.float64) - h[fin])
    assert np.all(err <= 1e-5 + 1e-5 * h[fin]), f"entropy max err {err.max():.3e}"
    assert np.array_equal(got["argmax"], ref["argmax"]), "greedy argmax ids differ"
    st = got["status"]
    if fin.any():
        assert abs(st["mean_entropy"] - ref["mean_entropy"]) <= 1e-5 + 1e-5 * ref["mean_entropy"]
    assert st["n_defined"] == int(fin.sum())
    rank = {int(pos): k for k, pos in enumerate(ref["order"])}
    diff = np.nonzero(got["accepted"].astype(bool) != ref["accepted"].astype(bool))[0]
    for pos in diff:
        k = rank[int(pos)]
        near_budget = abs(ref["csum"][k] - BUDGET) <= 1e-4
        others = np.delete(h[fin], np.searchsorted(np.nonzero(fin)[0], pos))
        near_tie = others.size > 0 and np.min(np.abs(others - h[pos])) <= 2e-5
        assert near_budget or near_tie, (f"position {pos}: accepted gpu={got['accepted'][pos]} "
                                         f"oracle={ref['accepted'][pos]} rank {k} csum {ref['csum'][k]}")
    assert st["n_accepted"] == int(got["accepted"].sum())
    if bool(st["stop"]) != ref["stop"]:
        assert abs(ref["mean_entropy"] - STOP) <= 1e-5, "stop flag differs away from the threshold"
        return len(diff) + 1
    if ref["stop"]:
        assert np.array_equal(got["ids"], ref["argmax"])
        return len(diff)
    both = got["accepted"].astype(bool) & ref["accepted"].astype(bool)
    neither = ~got["accepted"].astype(bool) & ~ref["accepted"].astype(bool)
    for pos in np.nonzero(both)[0]:
        if got["ids"][pos] != ref["cand"][pos]:
            assert ref["gap"][pos] <= BAND, f"position {pos}: candidate differs, gap {ref['gap'][pos]}"
    assert np.array_equal(got["ids"][neither], ref["ids"][neither]), "re-noise draws differ"
    return len(diff)


def spread_logits(rng, n, vocab, lo=6.0, hi=22.0, std=1.0):
    """Noise plus one spike per row whose height spreads the row entropies from
    near zero to several nats, so the budget cuts through the sorted order."""
    l = (rng.standard_normal((n, vocab)) * std).astype(np.float32)
    tgt = rng.integers(0, vocab, n)
    l[np.arange(n), tgt] += rng.uniform(lo, hi, n).astype(np.float32)
    return l


@pytest.mark.parametrize("n,vocab,d,flags", [
    (256, 4096, 512, 0),
    (256, 32768, 256, S.GUMBEL | S.T_SCHEDULE),
    (100, 5003, 64, S.T_SCHEDULE),
    (1, 1000, 8, 0),
    (256, 12345, 130, S.GUMBEL),
])
def test_eb_step_matches_oracle(n, vocab, d, flags):
    torch, dg = require_gpu()
    log(f"eb step n={n} V={vocab} d={d} flags={flags}")
    rng = np.random.default_rng(n * 7 + vocab)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    ctrl = S.Ctrl(seed=31, gstep=5, s_in_block=3, s_max=48, flags=flags | S.AUTO_ADVANCE,
                  t_start=0.8, t_end=0.4)
    dev = DevEb(torch, dg, emb, n, ctrl)
    logits = spread_logits(rng, n, vocab)
    ids = rng.integers(0, vocab, n)
    got = dev.step(to_dev(logits), ids)
    rows = np.unique(np.array([0, n // 3, n - 1]))
    ref = EB.eb_step(logits, emb.astype(np.float64), ids, ctrl, None, BUDGET, STOP, z_rows=rows)
    exempt = check_eb(ref, got)
    check_z(got["z"][rows], ref["z"])
    assert got["ctrl"]["gstep"] == 6 and got["ctrl"]["s_in_block"] == 4
    assert exempt <= 2
    log(f"  accepted {got['status']['n_accepted']} (oracle {ref['n_accepted']}), exempt {exempt}")


def test_eb_undefined_rows_and_last_step():
    torch, dg = require_gpu()
    rng = np.random.default_rng(41)
    n, vocab, d = 64, 3000, 32
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    logits = spread_logits(rng, n, vocab)
    logits[3, 17] = np.nan
    logits[9, :] = -np.inf
    logits[12, 5] = np.inf
    for s_in_block in (10, 47):
        ctrl = S.Ctrl(seed=5, gstep=s_in_block, s_in_block=s_in_block, s_max=48)
        dev = DevEb(torch, dg, emb, n, ctrl)
        ids = rng.integers(0, vocab, n)
        got = dev.step(to_dev(logits), ids)
        ref = EB.eb_step(logits, emb, ids, ctrl, None, BUDGET, STOP, z_rows=None)
        check_eb(ref, got)
        assert not got["accepted"][[3, 9, 12]].any()
        assert np.isnan(got["z"][[3, 9, 12]]).all()
        if s_in_block == 47:
            assert got["status"]["n_accepted"] == n - 3


def test_eb_canvas_adaptive_stop():
    """A canvas denoised to its stop on the device, logits made on the host from
    the device's ids each step; every step compared with the oracle."""
    torch, dg = require_gpu()
    n, vocab, d = 256, 32768, 128
    rng = np.random.default_rng(42)
    target = rng.integers(0, vocab, n)
    noise = (rng.standard_normal((n, vocab)) * 0.5).astype(np.float32)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)

    def make_logits(ids, s):
        l = noise.copy()
        boost = np.where(ids == target, 60.0, 8.0 + 2.0 * s).astype(np.float32)
        l[np.arange(n), target] += boost
        return l

    ctrl = S.Ctrl(seed=6, s_max=48, flags=S.T_SCHEDULE | S.AUTO_ADVANCE, t_start=0.8, t_end=0.4)
    ids, _, ctrl = S.init_canvas(ctrl, n, vocab)
    dev = DevEb(torch, dg, emb, n, ctrl)
    dev.ids.copy_(to_dev(ids.astype(np.int32)))
    prev = None
    for step in range(48):
        logits = make_logits(ids, ctrl.s_in_block)
        got = dev.step(to_dev(logits))
        ref = EB.eb_step(logits, emb, ids, ctrl, prev, BUDGET, STOP, z_rows=None)
        check_eb(ref, got)
        ids, prev, ctrl = got["ids"], got["argmax"], ref["ctrl"]
        if got["status"]["stop"]:
            break
    log(f"eb canvas stopped after {step + 1} steps")
    assert got["status"]["stop"] and step + 1 < 48
    assert np.array_equal(ids, target)


def test_eb_full_vocab_step():
    torch, dg = require_gpu()
    log("eb full vocabulary: drawing inputs")
    emb = workloads.embedding(3)
    n, vocab = 256, emb.shape[0]
    rng = np.random.default_rng(43)
    logits = spread_logits(rng, n, vocab, lo=8.0, hi=26.0, std=2.0)
    ctrl = S.Ctrl(seed=7, gstep=2, s_in_block=2, s_max=48, flags=S.GUMBEL | S.T_SCHEDULE,
                  t_start=0.8, t_end=0.4)
    dev = DevEb(torch, dg, emb, n, ctrl)
    ids = rng.integers(0, vocab, n)
    got = dev.step(to_dev(logits), ids)
    rows = np.array([0, 101, 255])
    ref = EB.eb_step(logits, emb.astype(np.float64), ids, ctrl, None, BUDGET, STOP, z_rows=rows)
    exempt = check_eb(ref, got)
    check_z(got["z"][rows], ref["z"])
    log(f"  accepted {got['status']['n_accepted']} (oracle {ref['n_accepted']}), exempt {exempt}")
    assert exempt <= 2
