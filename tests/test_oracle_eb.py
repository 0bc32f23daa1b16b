"""Pins for the oracle's entropy-bounded sampler and adaptive stopping (CPU only)."""
from dataclasses import replace

import numpy as np
import pytest
from scipy import stats

from oracle import eb
from oracle import philox
from oracle import sampler as S


@pytest.mark.parametrize("temp", [1.0, 0.8, 0.4])
def test_entropy_matches_scipy(temp):
    rng = np.random.default_rng(20)
    l = (rng.standard_normal((6, 777)) * 3).astype(np.float32)
    l[2, 5] += 25.0                                   # a nearly one-hot row
    ref = stats.entropy(np.exp((l.astype(np.float64) - l.max(1, keepdims=True)) / temp), axis=1)
    np.testing.assert_allclose(eb.entropy64(l, temp), ref, rtol=1e-12, atol=1e-15)


def test_entropy_closed_forms():
    v = 4096
    np.testing.assert_allclose(eb.entropy64(np.zeros((3, v), np.float32), 0.7), np.log(v), rtol=1e-14)
    a, b, t = 1.3, -0.9, 0.6
    l = np.full((1, 5), -np.inf, np.float32)
    l[0, 1], l[0, 3] = a, b
    q = 1.0 / (1.0 + np.exp(-(np.float64(np.float32(a)) - np.float64(np.float32(b))) / t))
    h2 = -(q * np.log(q) + (1 - q) * np.log(1 - q))
    np.testing.assert_allclose(eb.entropy64(l, t), [h2], rtol=1e-13)


def test_acceptance_budget_cases():
    acc, order, csum = eb.accept_order(np.array([0.05, 0.01, 0.03, 0.02, np.nan]))
    assert list(order) == [1, 3, 2, 0]
    assert acc.tolist() == [False, True, True, True, False]
    acc, _, _ = eb.accept_order(np.array([0.05, 0.05]))          # inclusive at the budget
    assert acc.tolist() == [True, True]
    acc, _, _ = eb.accept_order(np.array([6.0, 5.0, 7.0]))       # at least one: the lowest
    assert acc.tolist() == [False, True, False]
    acc, order, _ = eb.accept_order(np.array([0.04, 0.04, 0.04]))  # ties by position
    assert list(order) == [0, 1, 2] and acc.tolist() == [True, True, False]
    acc, order, _ = eb.accept_order(np.array([np.nan, np.nan]))
    assert not acc.any() and len(order) == 0


def _spiky(n, vocab, heights, rng):
    l = (rng.standard_normal((n, vocab)) * 1.0).astype(np.float32)
    tgt = rng.integers(0, vocab, n)
    l[np.arange(n), tgt] += np.asarray(heights, np.float32)
    return l, tgt


def test_step_accepts_low_entropy_and_renoises_the_rest():
    rng = np.random.default_rng(21)
    n, vocab = 32, 2048
    heights = np.where(np.arange(n) % 4 == 0, 40.0, 0.0)        # 8 near-certain rows
    l, tgt = _spiky(n, vocab, heights, rng)
    ctrl = S.Ctrl(seed=9, gstep=3, tau=0.9)
    e = np.eye(vocab, 4, dtype=np.float32)
    ids = rng.integers(0, vocab, n)
    r = eb.eb_step(l, e, ids, ctrl)
    sure = np.arange(n) % 4 == 0
    assert r["accepted"][sure].all() and not r["accepted"][~sure].any()
    assert np.array_equal(r["ids"][sure], tgt[sure])
    draws = philox.renoise_ids(9, 3, np.arange(n), vocab)
    assert np.array_equal(r["ids"][~sure], draws[~sure])
    assert r["n_accepted"] == 8 and not r["stop"]


def test_previously_accepted_positions_are_redecided():
    rng = np.random.default_rng(22)
    n, vocab = 8, 512
    l1, t1 = _spiky(n, vocab, [40, 0, 0, 0, 0, 0, 0, 0], rng)
    ctrl = S.Ctrl(seed=1, gstep=0, tau=0.9, flags=S.AUTO_ADVANCE)
    r1 = eb.eb_step(l1, None, rng.integers(0, vocab, n), ctrl, z_rows=None)
    assert r1["accepted"][0] and r1["ids"][0] == t1[0]
    l2, t2 = _spiky(n, vocab, [0, 40, 0, 0, 0, 0, 0, 0], rng)
    r2 = eb.eb_step(l2, None, r1["ids"], r1["ctrl"], prev_argmax=r1["argmax"], z_rows=None)
    assert not r2["accepted"][0] and r2["accepted"][1]
    assert r2["ids"][0] == philox.renoise_ids(1, 1, [0], vocab)[0]


def test_stop_rule_truth_table():
    rng = np.random.default_rng(23)
    n, vocab = 16, 1024
    l, tgt = _spiky(n, vocab, np.full(n, 60.0), rng)              # every row near-certain
    ctrl = S.Ctrl(seed=2, gstep=5)
    first = eb.eb_step(l, None, tgt, ctrl, prev_argmax=None, z_rows=None)
    assert first["mean_entropy"] < eb.STOP_ENTROPY and not first["stop"]   # no previous step
    same = eb.eb_step(l, None, tgt, ctrl, prev_argmax=tgt, z_rows=None)
    assert same["stop"] and np.array_equal(same["ids"], tgt)               # E5
    moved = tgt.copy(); moved[3] = (moved[3] + 1) % vocab
    assert not eb.eb_step(l, None, tgt, ctrl, prev_argmax=moved, z_rows=None)["stop"]
    flat = np.zeros((n, vocab), np.float32)
    r = eb.eb_step(flat, None, tgt, ctrl, prev_argmax=np.zeros(n, np.int64), z_rows=None)
    assert r["mean_entropy"] == pytest.approx(np.log(vocab)) and not r["stop"]
    assert r["n_accepted"] == 1 and r["accepted"][0]                       # at least one, lowest position


def test_last_step_accepts_every_defined_row():
    rng = np.random.default_rng(24)
    n, vocab = 8, 256
    l = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    l[5, 7] = np.nan
    ctrl = S.Ctrl(seed=3, gstep=47, s_in_block=47, s_max=48)
    r = eb.eb_step(l, None, np.zeros(n, np.int64), ctrl, z_rows=None)
    assert r["accepted"].tolist() == [1, 1, 1, 1, 1, 0, 1, 1]
    assert np.isnan(r["entropy"][5]) and np.array_equal(r["ids"][r["accepted"] == 1], r["cand"][r["accepted"] == 1])


def test_canvas_converges_with_adaptive_stopping():
    """A generator that grows more certain as positions are accepted: the canvas
    must stop before the budget with the stable prediction as its ids."""
    n, vocab = 64, 4096
    rng = np.random.default_rng(25)
    target = rng.integers(0, vocab, n)
    noise = (rng.standard_normal((n, vocab)) * 0.5).astype(np.float32)

    def logits(ids, ctrl):
        l = noise.copy()
        hit = (ids == target)
        boost = np.where(hit, 60.0, 8.0 + 2.0 * ctrl.s_in_block).astype(np.float32)
        l[np.arange(n), target] += boost
        return l

    ctrl = S.Ctrl(seed=4, s_max=48, flags=S.T_SCHEDULE, t_start=0.8, t_end=0.4)
    ids, steps, _ = eb.eb_canvas(logits, None, ctrl, n, vocab)
    assert steps[-1]["stop"] and len(steps) < 48
    assert np.array_equal(ids, target)
