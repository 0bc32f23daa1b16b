"""The merges a sharded step would rely on, checked on the CPU against the oracle.

A step split over several devices (by vocabulary for the sampler, by keys for
attention) needs each shard to reduce its part to a few numbers and a partial
vector, and one merge to give the unsharded result.  The one-device kernels
already do this across their own splits (the sampler's statistics and partial z
per split, attention's per-chunk (m, l, O)); these tests check the same merge
across shards of uneven size, including empty shards and shards whose ids all
have probability zero, against the oracle's unsharded definitions:
  - z = softmax(l)·E (DiffusionGemma Technical Report part 4/6, section 6
    "Sampling", self-conditioning) from per-shard (max, sum, partial z);
  - the greedy candidate (the argmax of the row, lowest id on ties) from
    per-shard argmaxes;
  - canvas attention (section 6 "Attention") from per-key-shard (m, l, O).
No GPU and no library code: numpy and the oracle only.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import sampler as OS


def _bounds(total, cuts):
    edges = [0] + sorted(cuts) + [total]
    return list(zip(edges[:-1], edges[1:]))


def _vocab_shard(l, emb, lo, hi):
    """One shard's statistics: max, sum of exp(l - max), partial z, argmax."""
    part = l[:, lo:hi]
    n = l.shape[0]
    if hi == lo:
        return np.full(n, -np.inf), np.zeros(n), np.zeros((n, emb.shape[1])), np.full(n, -1)
    m = part.max(axis=1)
    w = np.where(np.isfinite(m)[:, None], np.exp(part - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
    return m, w.sum(axis=1), w @ emb[lo:hi], lo + np.argmax(part, axis=1)


def _vocab_merge(shards):
    ms = np.stack([s[0] for s in shards])                  # [G, N]
    m = ms.max(axis=0)
    f = np.where(np.isfinite(ms), np.exp(ms - m), 0.0)     # weight of each shard
    s = (f * np.stack([s[1] for s in shards])).sum(axis=0)
    z = np.einsum("gn,gnd->nd", f, np.stack([s[2] for s in shards])) / s[:, None]
    # argmax: the largest shard maximum, the lowest shard (so the lowest id) on ties
    best = np.argmax(ms, axis=0)
    ids = np.stack([s[3] for s in shards])[best, np.arange(ms.shape[1])]
    return z, ids


@pytest.mark.parametrize("cuts", [[], [1000], [17, 2500, 2501, 4000], [0, 0, 4099]])
def test_vocab_shards_merge_to_the_unsharded_sampler(cuts):
    rng = np.random.default_rng(len(cuts) + 1)
    n, vocab, d = 24, 4099, 40
    l = rng.standard_normal((n, vocab)) * 2.0
    l[::3, 1234] += 12.0                                   # peaked rows
    l[1, 2000:2600] = -np.inf                              # a shard-sized stretch of zero probability
    l[2, 7] = l[2, 3001] = l[2].max() + 1.0                # a tie across shards: id 7 must win
    emb = rng.standard_normal((vocab, d)) * 0.02
    z, ids = _vocab_merge([_vocab_shard(l, emb, lo, hi) for lo, hi in _bounds(vocab, cuts)])
    np.testing.assert_allclose(z, OS.selfcond(l, emb), rtol=0, atol=1e-13)
    assert ids[2] == 7
    np.testing.assert_array_equal(ids, np.argmax(l, axis=1))


def test_vocab_merge_detects_a_dropped_shard_weight():
    """The check is sharp: merging without the exp(m_g - m) weights fails it."""
    rng = np.random.default_rng(5)
    n, vocab, d = 8, 600, 16
    l = rng.standard_normal((n, vocab)) * 3.0
    emb = rng.standard_normal((vocab, d)) * 0.02
    shards = [_vocab_shard(l, emb, lo, hi) for lo, hi in _bounds(vocab, [200, 400])]
    bad = sum(s[2] for s in shards) / sum(s[1] for s in shards)[:, None]
    assert np.abs(bad - OS.selfcond(l, emb)).max() > 1e-4


def _key_shard(q, keys, vals, lo, hi, scale):
    """Per key shard, per (row, query head): max score, sum of weights, unnormalised O."""
    n, hq, d = q.shape
    g = hq // keys.shape[1]
    m = np.full((n, hq), -np.inf)
    lsum = np.zeros((n, hq))
    o = np.zeros((n, hq, d))
    if hi == lo:
        return m, lsum, o
    for h in range(hq):
        s = scale * (q[:, h, :] @ keys[lo:hi, h // g, :].T)
        m[:, h] = s.max(axis=1)
        w = np.exp(s - m[:, h][:, None])
        lsum[:, h] = w.sum(axis=1)
        o[:, h, :] = w @ vals[lo:hi, h // g, :]
    return m, lsum, o


@pytest.mark.parametrize("cuts", [[], [64], [5, 300, 301], [0, 420]])
def test_key_shards_merge_to_the_unsharded_attention(cuts):
    rng = np.random.default_rng(len(cuts) + 11)
    n, p, hq, hkv, d = 20, 400, 4, 2, 32
    q = rng.standard_normal((n, hq, d))
    kp, vp = rng.standard_normal((p, hkv, d)), rng.standard_normal((p, hkv, d))
    kc, vc = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    keys, vals = np.concatenate([kp, kc]), np.concatenate([vp, vc])
    scale = 1.0 / np.sqrt(d)
    parts = [_key_shard(q, keys, vals, lo, hi, scale) for lo, hi in _bounds(p + n, cuts)]
    ms = np.stack([x[0] for x in parts])
    m = ms.max(axis=0)
    f = np.where(np.isfinite(ms), np.exp(ms - m), 0.0)
    lsum = (f * np.stack([x[1] for x in parts])).sum(axis=0)
    o = np.einsum("gnh,gnhd->nhd", f, np.stack([x[2] for x in parts])) / lsum[..., None]
    np.testing.assert_allclose(o, OA.canvas_attention(q, kp, vp, kc, vc), rtol=0, atol=1e-12)
