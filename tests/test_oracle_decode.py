"""Pins for the synthetic decode run: generator behaviour, canvas completion, resume identity (CPU only)."""
from dataclasses import replace

import numpy as np
import pytest

import workloads
from oracle import decode, sampler as S, synth


def _blocks(n_blocks, n=256, hkv=2, d=16):
    rng = np.random.default_rng(0)
    return [dict(q=rng.standard_normal((n, 4, d)), k_canvas=rng.standard_normal((n, hkv, d)),
                 v_canvas=rng.standard_normal((n, hkv, d))) for _ in range(n_blocks)]


CTRL5 = S.Ctrl(seed=5, tau=0.9, s_max=48, flags=S.GUMBEL | S.T_SCHEDULE | S.AUTO_ADVANCE,
               t_start=0.8, t_end=0.4)


def test_canvas_completes_at_about_20_per_step():
    vocab = 8192
    table = workloads.synth_table()
    recs, ctrl = decode.decode_run(np.zeros((8, 2, 16)), np.zeros((8, 2, 16)), _blocks(1), None,
                                   table, vocab, CTRL5, z_rows=None, with_attention=False)
    steps = recs[0]["steps"]
    n_unc = [s["n_uncommitted"] for s in steps]
    assert n_unc[-1] == 0
    accepted = -np.diff([256] + n_unc)
    # the generator chooses about 20 open rows per step; every chosen row commits
    assert 10 <= len(steps) <= 18, len(steps)
    assert abs(np.mean(accepted[:-1]) - 20) < 6
    # commits are monotone and never revisited
    prev = np.zeros(256, np.uint8)
    prev_ids = None
    for s in steps:
        assert np.all(s["committed"] >= prev)
        if prev_ids is not None:
            keep = prev.astype(bool)
            assert np.all(s["ids"][keep] == prev_ids[keep])
        prev, prev_ids = s["committed"], s["ids"]
    assert ctrl.gstep == len(steps)


def test_noise_rows_stay_below_threshold_at_full_vocab():
    vocab = 262144
    table = workloads.synth_table()
    ids = np.zeros(256, np.int64)
    mask = np.zeros(256, np.uint8)
    l = synth.synth_logits(ids, mask, gstep=0, seed=5, table=table, vocab=vocab, rows=np.arange(6))
    for temp in (1.0, 0.8, 0.4):
        p = S.softmax64(l, temp)
        top = p.max(axis=1)
        spiked = top > 0.5
        assert np.all(top[~spiked] < 0.015)
        assert np.all(top[spiked] > 0.999)


def test_resume_identity():
    vocab = 4096
    table = workloads.synth_table()
    kp = np.random.default_rng(1).standard_normal((16, 2, 16))
    blocks = _blocks(2)
    full, ctrl_full = decode.decode_run(kp, kp, blocks, None, table, vocab, CTRL5, with_attention=True)
    first, ctrl_mid = decode.decode_run(kp, kp, blocks[:1], None, table, vocab, CTRL5, with_attention=True)
    kp2 = np.concatenate([kp, blocks[0]["k_canvas"]])
    vp2 = np.concatenate([kp, blocks[0]["v_canvas"]])
    second, ctrl_end = decode.decode_run(kp2, vp2, blocks[1:], None, table, vocab,
                                         replace(ctrl_mid), with_attention=True)
    assert ctrl_end == ctrl_full
    np.testing.assert_array_equal(full[1]["final_ids"], second[0]["final_ids"])
    np.testing.assert_array_equal(full[1]["attention"], second[0]["attention"])
    assert full[1]["n_prefix"] == 16 + 256


def test_synth_spike_is_one_float32_add():
    from oracle import philox
    table = workloads.synth_table()
    vocab = 4096
    ids = np.arange(256) * 13
    mask = np.zeros(256, np.uint8); mask[::2] = 1
    l = synth.synth_logits(ids, mask, gstep=3, seed=5, table=table, vocab=vocab, rows=np.arange(4))
    jj = np.arange(vocab, dtype=np.uint64)
    for r in range(4):
        h = philox.word(5, philox.STREAM_SYN_NOISE, 3, r, c0=jj >> np.uint64(2),
                        w=(jj & np.uint64(3)).astype(np.int64))
        noise = table[(h >> np.uint32(16)).astype(np.int64)]
        diff = np.nonzero(l[r] != noise)[0]
        if mask[r]:
            assert list(diff) == [ids[r]]
            assert l[r, ids[r]] == np.float32(noise[ids[r]] + np.float32(30))
        else:
            assert len(diff) <= 1
            if len(diff):
                assert l[r, diff[0]] == np.float32(noise[diff[0]] + np.float32(30))
