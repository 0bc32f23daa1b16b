"""Pins for the oracle's top-k truncation of the sampler step (CPU only)."""

import numpy as np
import pytest
import torch
from scipy import special, stats

from oracle import eb as EB
from oracle import sampler as S
from oracle import topk as K


def brute_keep(row, k):
    """An id is kept iff fewer than k ids come before it (larger value, or the
    same value and a smaller id)."""
    v = len(row)
    keep = np.zeros(v, dtype=bool)
    for j in range(v):
        before = sum(1 for i in range(v) if row[i] > row[j] or (row[i] == row[j] and i < j))
        keep[j] = before < k
    return keep


def test_keep_set_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for _ in range(200):
        v = int(rng.integers(1, 9))
        row = rng.integers(-2, 3, v).astype(np.float32)      # many ties
        if rng.random() < 0.2:
            row[rng.integers(0, v)] = -np.inf
        for k in range(1, v + 2):
            assert np.array_equal(K.keep_mask(row, k), brute_keep(row, k)), (row, k)


def test_keep_set_matches_torch_topk_on_distinct_values():
    rng = np.random.default_rng(1)
    l = rng.permutation(5000).reshape(5, 1000).astype(np.float32) * 0.01
    for k in (1, 7, 64, 256, 999):
        idx = torch.topk(torch.from_numpy(l), k, dim=1).indices.numpy()
        for i in range(5):
            want = np.zeros(1000, bool)
            want[idx[i]] = True
            assert np.array_equal(K.keep_mask(l[i], k), want)


@pytest.mark.parametrize("temp", [1.0, 0.6])
def test_truncated_softmax_is_renormalised_full_softmax(temp):
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((6, 700)) * 3).astype(np.float32)
    k = 50
    lt = K.truncate_top_k(l, k)
    p_full = special.softmax(l.astype(np.float64) / temp, axis=1)
    p_trunc = S.softmax64(lt, temp)
    for i in range(6):
        keep = K.keep_mask(l[i], k)
        want = np.where(keep, p_full[i], 0.0) / p_full[i][keep].sum()
        np.testing.assert_allclose(p_trunc[i], want, rtol=1e-12, atol=1e-300)
        assert np.count_nonzero(p_trunc[i]) == k


def test_k_one_is_one_hot():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((5, 300)) * 2).astype(np.float32)
    e = rng.standard_normal((300, 9)).astype(np.float32)
    ctrl = S.Ctrl(seed=4, tau=0.999)
    r = K.sampler_step_topk(l, e, np.zeros(5, int), np.zeros(5, np.uint8), ctrl, 1)
    am = np.argmax(l, axis=1)
    np.testing.assert_array_equal(r["z"], e[am].astype(np.float64))
    np.testing.assert_array_equal(r["kappa"], 1.0)
    assert r["committed"].all() and np.array_equal(r["ids"], am)


def test_equal_logits_keep_first_ids():
    e = np.random.default_rng(4).standard_normal((40, 6)).astype(np.float32)
    l = np.zeros((2, 40), np.float32)
    k = 8
    lt = K.truncate_top_k(l, k)
    assert np.all(np.isfinite(lt[:, :k])) and np.all(np.isneginf(lt[:, k:]))
    z = S.selfcond(lt, e)
    np.testing.assert_allclose(z, np.broadcast_to(e[:k].astype(np.float64).mean(0), (2, 6)), rtol=1e-14)
    h = EB.entropy64(np.where(np.isneginf(lt), -np.inf, lt), 1.0)
    np.testing.assert_allclose(h, np.log(k), rtol=1e-14)


def test_k_at_least_vocab_changes_nothing():
    rng = np.random.default_rng(5)
    l = (rng.standard_normal((8, 64)) * 3).astype(np.float32)
    e = rng.standard_normal((64, 5)).astype(np.float32)
    ids = rng.integers(0, 64, 8)
    mask = (rng.random(8) < 0.3).astype(np.uint8)
    ctrl = S.Ctrl(seed=9, gstep=2, flags=S.GUMBEL, t_start=0.7, t_end=0.7, tau=0.3)
    full = S.sampler_step(l, e, ids, mask, ctrl)
    for k in (64, 65, 1000):
        r = K.sampler_step_topk(l, e, ids, mask, ctrl, k)
        for key in ("ids", "committed", "z", "kappa", "cand"):
            np.testing.assert_array_equal(r[key], full[key])


def test_undefined_rows_stay_undefined_and_short_rows_keep_weight_zero():
    l = np.full((3, 20), -np.inf, np.float32)
    l[0, 3] = np.nan
    l[1, :] = -np.inf
    l[2, [4, 9]] = [1.0, 2.0]            # two finite logits, k = 5
    lt = K.truncate_top_k(l, 5)
    assert np.isnan(lt[0, 3]) and np.all(np.isneginf(lt[1]))
    assert list(np.nonzero(np.isfinite(lt[2]))[0]) == [4, 9]
    bad = S.undefined_rows(lt)
    assert list(bad) == [True, True, False]
    p = S.softmax64(np.where(bad[:, None], 0.0, lt.astype(np.float64)))[2]
    np.testing.assert_allclose(p[[4, 9]], special.softmax([1.0, 2.0]), rtol=1e-14)


def test_gumbel_candidates_stay_in_the_kept_set_and_follow_truncated_p():
    temp = 0.7
    logits = np.array([0.0, 0.9, -0.2, 0.6, 0.1, -1.0, 0.8], np.float32)
    k = 3
    n = 6000
    l = np.broadcast_to(logits, (n, 7)).copy()
    ctrl = S.Ctrl(seed=13, flags=S.GUMBEL, t_start=temp, t_end=temp)
    cand, _ = S.candidates(K.truncate_top_k(l, k), ctrl, S.temperature(ctrl))
    keep = K.keep_mask(logits, k)
    assert np.all(keep[cand])
    p = special.softmax(np.where(keep, logits.astype(np.float64), -np.inf) / float(np.float32(temp)))
    kept = np.nonzero(keep)[0]
    counts = np.bincount(cand, minlength=7)[kept]
    _, pval = stats.chisquare(counts, p[kept] * n)
    assert pval > 1e-4


def test_entropy_bounded_step_on_truncated_rows():
    rng = np.random.default_rng(6)
    l = (rng.standard_normal((10, 200)) * 0.5).astype(np.float32)
    l[np.arange(10), rng.integers(0, 200, 10)] += np.linspace(2, 12, 10).astype(np.float32)
    e = rng.standard_normal((200, 4)).astype(np.float32)
    ctrl = S.Ctrl(seed=3, s_max=48)
    k = 16
    r = K.eb_step_topk(l, e, rng.integers(0, 200, 10), ctrl, k)
    for i in range(10):
        keep = K.keep_mask(l[i], k)
        want = stats.entropy(special.softmax(l[i][keep].astype(np.float64)))
        np.testing.assert_allclose(r["entropy"][i], want, rtol=1e-12)
    # truncation removes tail mass, so every row's entropy drops
    full = EB.entropy64(l, 1.0)
    assert np.all(r["entropy"] < full)
