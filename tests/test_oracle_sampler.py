"""Pins for the oracle's sampler step (CPU only)."""
import json
import os
from dataclasses import replace

import numpy as np
import pytest
from scipy import special, stats

from oracle import philox
from oracle import sampler as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    l = rng.standard_normal((7, 513)).astype(np.float32) * 5
    np.testing.assert_allclose(S.softmax64(l), special.softmax(l.astype(np.float64), axis=1), rtol=1e-13)
    np.testing.assert_allclose(S.softmax64(l, 0.4), special.softmax(l.astype(np.float64) / 0.4, axis=1), rtol=1e-12)
    # log of the normaliser against scipy's logsumexp
    p = S.softmax64(l)
    lse = special.logsumexp(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.log(p[:, 0]), l[:, 0] - lse, rtol=1e-12, atol=1e-12)


def test_selfcond_identity_embedding_gives_probabilities():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((16, 64)).astype(np.float32) * 3
    z = S.selfcond(l, np.eye(64, dtype=np.float32))
    np.testing.assert_allclose(z, special.softmax(l.astype(np.float64), axis=1), rtol=1e-13)


def test_selfcond_ones_column_sums_to_one():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((8, 1000)).astype(np.float32) * 4
    e = rng.standard_normal((1000, 5)).astype(np.float32)
    e[:, 3] = 1
    z = S.selfcond(l, e)
    np.testing.assert_allclose(z[:, 3], 1.0, rtol=0, atol=1e-14)


def test_selfcond_uniform_and_spike_and_linearity():
    rng = np.random.default_rng(3)
    e = rng.standard_normal((300, 12)).astype(np.float32)
    z = S.selfcond(np.zeros((2, 300), np.float32), e)
    np.testing.assert_allclose(z, np.broadcast_to(e.astype(np.float64).mean(0), (2, 12)), atol=1e-14)
    l = rng.standard_normal((3, 300)).astype(np.float32)
    l[np.arange(3), [5, 77, 299]] += 100
    z = S.selfcond(l, e)
    np.testing.assert_allclose(z, e[[5, 77, 299]].astype(np.float64), rtol=1e-30, atol=1e-30 + 1e-35)
    e2 = rng.standard_normal((300, 12)).astype(np.float32)
    np.testing.assert_allclose(S.selfcond(l, e) * 2 - S.selfcond(l, e2),
                               S.selfcond(l, 2 * e.astype(np.float64) - e2), atol=1e-12)


@pytest.mark.parametrize("temp", [1.0, 0.8, 0.4])
def test_two_logit_closed_form(temp):
    a, b = 1.7, -0.4
    l = np.array([[a, b]], np.float32)
    ctrl = S.Ctrl(t_start=temp, t_end=temp, tau=0.99)
    res = S.sampler_step(l, np.eye(2, dtype=np.float32), [0], [0], ctrl, z_rows=None)
    t = float(np.float32(temp))
    expect = 1 / (1 + np.exp(-(float(np.float32(a)) - float(np.float32(b))) / t))
    assert res["cand"][0] == 0
    np.testing.assert_allclose(res["kappa"][0], expect, rtol=1e-14)


def test_temperature_schedule_table2():
    g = json.load(open(os.path.join(GOLDEN, "table2_sampler_hparams.json")))
    c = S.Ctrl(flags=S.T_SCHEDULE, s_max=g["max_denoising_steps"],
               t_start=g["temperature_start"], t_end=g["temperature_end"])
    ts = [float(S.temperature(replace(c, s_in_block=s))) for s in range(g["max_denoising_steps"])]
    assert ts[0] == pytest.approx(g["temperature_start"], abs=1e-7)
    assert ts[-1] == pytest.approx(g["temperature_end"], abs=1e-7)
    assert np.all(np.diff(ts) < 0)
    np.testing.assert_allclose(np.diff(ts), -0.4 / 47, rtol=1e-4)
    # without the schedule flag the temperature is t_start at every step
    assert float(S.temperature(replace(c, flags=0, s_in_block=30))) == pytest.approx(0.8, abs=1e-7)


def test_gumbel_candidates_sample_p_t():
    # the Gumbel candidate is a draw from softmax(l / T): chi-square over positions
    temp = 0.5
    logits = np.array([0.0, 0.3, -0.2, 0.6, 0.1, -1.0], np.float32)
    n = 6000
    l = np.broadcast_to(logits, (n, 6)).copy()
    ctrl = S.Ctrl(seed=99, flags=S.GUMBEL, t_start=temp, t_end=temp, tau=2.0)
    cand, _ = S.candidates(l, ctrl, S.temperature(ctrl))
    p = special.softmax(logits.astype(np.float64) / float(np.float32(temp)))
    chi2, pval = stats.chisquare(np.bincount(cand, minlength=6), p * n)
    assert pval > 1e-4


@pytest.mark.parametrize("temp", [1.0, 0.8, 0.4])
@pytest.mark.parametrize("a,b", [(1.7, -0.4), (-3.0, 2.25), (0.5, 0.5), (12.0, -7.5)])
def test_greedy_gap_two_logit_closed_form(temp, a, b):
    """Greedy mode: the top-2 gap is in probability units of p_T.  For two logits
    p_T = (sigma((a-b)/T), sigma((b-a)/T)), so the gap is |2 sigma((a-b)/T) - 1|
    = |tanh((a - b) / (2T))|, with T the float32 temperature."""
    l = np.array([[a, b]], np.float32)
    ctrl = S.Ctrl(t_start=temp, t_end=temp)
    t32 = S.temperature(ctrl)
    cand, gap = S.candidates(l, ctrl, t32)
    a32, b32 = float(l[0, 0]), float(l[0, 1])
    want = abs(np.tanh((a32 - b32) / (2.0 * float(t32))))
    np.testing.assert_allclose(gap[0], want, rtol=1e-12, atol=1e-15)
    assert cand[0] == (0 if a32 >= b32 else 1)


def test_greedy_gap_three_logit_closed_form():
    """Three logits a > b > c at temperature T: gap = (1 - e^{(b-a)/T}) /
    (1 + e^{(b-a)/T} + e^{(c-a)/T}), which no two-logit case distinguishes
    from a gap taken at T = 1 or over the raw logits."""
    a, b, c, temp = 2.0, 1.25, -0.5, 0.4
    l = np.array([[c, a, b]], np.float32)
    ctrl = S.Ctrl(t_start=temp, t_end=temp)
    t = float(S.temperature(ctrl))
    _, gap = S.candidates(l, ctrl, S.temperature(ctrl))
    eb, ec = np.exp((b - a) / t), np.exp((c - a) / t)
    np.testing.assert_allclose(gap[0], (1 - eb) / (1 + eb + ec), rtol=1e-12)


@pytest.mark.parametrize("temp", [1.0, 0.5])
def test_gumbel_gap_is_in_score_units(temp):
    """Gumbel mode: the gap is the difference of the two best perturbed scores
    l_j / T + g_j, with g_j = -ln(-ln u_j) from the Philox word of id j (stream
    0, counter (j >> 2, position, gstep, 0), word j & 3) and u_j = (2 (h >> 9) + 1)
    2^-24.  The scores are computed here in float64 from those words; the oracle
    takes them in float32, so they agree to float32 rounding."""
    seed, gstep, pos = 77, 5, 3
    l = np.full((pos + 1, 5), -1.0, np.float32)
    l[pos] = np.array([10.0, 0.0, 0.25, -2.0, 9.5], np.float32)
    ctrl = S.Ctrl(seed=seed, gstep=gstep, flags=S.GUMBEL, t_start=temp, t_end=temp)
    t32 = S.temperature(ctrl)
    cand, gap = S.candidates(l, ctrl, t32)
    k0, k1 = seed & 0xFFFFFFFF, seed >> 32
    scores = []
    for j in range(5):
        words = philox.philox4x32_10(j >> 2, pos, gstep, 0, k0, k1)
        h = int(words[j & 3])
        u = (2 * (h >> 9) + 1) * 2.0 ** -24
        g = -np.log(-np.log(u))
        scores.append(float(l[pos, j]) / float(t32) + g)
    order = np.argsort(scores)[::-1]
    assert cand[pos] == order[0]
    np.testing.assert_allclose(gap[pos], scores[order[0]] - scores[order[1]], rtol=0, atol=1e-5)
    if temp == 0.5:
        # 10 / 0.5 against at most 9.5 / 0.5: a gap of this size exists only in score units
        assert gap[pos] > 1.0 or scores[order[1]] > 15


def test_greedy_ties_go_to_smallest_id():
    l = np.zeros((3, 10), np.float32)
    l[0, [4, 7]] = 5
    l[1, [9, 2, 3]] = 1
    l[2, :] = -1
    cand, gap = S.candidates(l, S.Ctrl(), np.float32(1))
    assert list(cand) == [4, 2, 0]
    assert np.all(gap == 0)


def test_commit_and_renoise_rules():
    rng = np.random.default_rng(4)
    n, vocab = 64, 500
    l = rng.standard_normal((n, vocab)).astype(np.float32)
    spike_rows = np.arange(0, n, 3)
    l[spike_rows, (spike_rows * 7) % vocab] += 40    # kappa ~ 1
    ids = rng.integers(0, vocab, n)
    mask = np.zeros(n, np.uint8)
    mask[[1, 2, 10]] = 1
    ctrl = S.Ctrl(seed=3, gstep=11, tau=0.9, flags=S.AUTO_ADVANCE)
    res = S.sampler_step(l, rng.standard_normal((vocab, 4)).astype(np.float32), ids, mask, ctrl)
    # committed on entry: untouched
    assert np.all(res["ids"][[1, 2, 10]] == ids[[1, 2, 10]])
    # spike rows that were open commit their spike id
    open_spikes = [r for r in spike_rows if mask[r] == 0]
    assert np.all(res["committed"][open_spikes] == 1)
    assert np.all(res["ids"][open_spikes] == (np.array(open_spikes) * 7) % vocab)
    # every other open row is renoised from the RENOISE stream at this step
    others = [r for r in range(n) if mask[r] == 0 and r not in set(open_spikes)]
    assert np.all(res["committed"][others] == 0)
    np.testing.assert_array_equal(res["ids"][others], philox.renoise_ids(3, 11, np.array(others), vocab))
    assert np.all(res["committed"] >= mask)                 # monotone mask
    assert res["n_uncommitted"] == len(others)
    assert res["ctrl"].gstep == 12 and res["ctrl"].s_in_block == 1
    # uniform rows never commit (kappa = 1/V)
    u = S.sampler_step(np.zeros((4, vocab), np.float32), np.eye(vocab, 2, dtype=np.float32), [0] * 4,
                       [0] * 4, ctrl, z_rows=None)
    np.testing.assert_allclose(u["kappa"], 1 / vocab)
    assert u["committed"].sum() == 0


def test_commit_only_changes_only_new_commits():
    rng = np.random.default_rng(5)
    n, vocab = 40, 300
    l = rng.standard_normal((n, vocab)).astype(np.float32)
    l[:10, 0] += 50
    ids = rng.integers(1, vocab, n)
    mask = np.zeros(n, np.uint8); mask[5:15] = 1
    res = S.sampler_step(l, np.ones((vocab, 1), np.float32), ids, mask,
                         S.Ctrl(flags=S.COMMIT_ONLY), z_rows=None)
    changed = res["ids"] != ids
    assert set(np.nonzero(changed)[0]) == set(range(5))
    assert np.all(res["committed"][:15] == 1) and res["committed"][15:].sum() == 0


def test_threshold_is_inclusive_in_float32():
    # kappa exactly 0.75 with V=2 at T=1: logits log(3), 0 -> p = 3/4
    l = np.array([[np.log(3.0), 0.0]], np.float32)
    t = float(1 / (1 + np.exp(-(np.float64(np.float32(np.log(3.0)))))))
    res = S.sampler_step(l, np.eye(2, dtype=np.float32), [1], [0], S.Ctrl(tau=np.float32(t)), z_rows=None)
    assert res["committed"][0] == 1


def test_forced_commit_on_last_step():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((10, 50)).astype(np.float32)
    ctrl = S.Ctrl(s_max=4, s_in_block=2, tau=0.99)
    assert S.sampler_step(l, np.eye(50, 3, dtype=np.float32), np.zeros(10), np.zeros(10), ctrl,
                          z_rows=None)["committed"].sum() == 0
    res = S.sampler_step(l, np.eye(50, 3, dtype=np.float32), np.zeros(10), np.zeros(10),
                         replace(ctrl, s_in_block=3), z_rows=None)
    assert res["committed"].sum() == 10
    np.testing.assert_array_equal(res["ids"], np.argmax(l, axis=1))


def test_undefined_rows():
    l = np.zeros((4, 8), np.float32)
    l[0, 3] = np.nan
    l[1, :] = -np.inf
    l[2, 1] = np.inf
    l[3, 5] = 9
    e = np.ones((8, 2), np.float32)
    res = S.sampler_step(l, e, [0, 0, 0, 0], [0, 0, 0, 0], S.Ctrl(tau=0.5, s_max=1))
    assert list(res["undefined"]) == [True, True, True, False]
    assert np.all(np.isnan(res["kappa"][:3])) and np.all(np.isnan(res["z"][:3]))
    assert list(res["committed"]) == [0, 0, 0, 1]       # even on the forced last step
    np.testing.assert_allclose(res["z"][3], [1, 1], atol=1e-14)
