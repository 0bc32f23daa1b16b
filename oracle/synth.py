"""Synthetic stand-in for the model's logits in the decode run (oracle side; test infrastructure only).

The pages' decode workload is a 4096-token input / 1024-token output request
(DiffusionGemma Technical Report, section 6 "Throughput for batch size of 1
serving", Eq. 12) at about 20 tokens per forward pass (explainer "DiffusionGemma:
Google's open diffusion LLM", section "About 20 tokens per pass against
speculative decoding").  Without weights, the logits come from this generator,
tuned so that the threshold sampler accepts about 20 positions per step:

  noise     l[i, j] = TN[h_noise >> 16], h_noise = word (j & 3) of
            counter (j >> 2, i, gstep, SYN_NOISE); TN is a 65536-entry float32
            table of N(0, 1) draws supplied as an input.
  chosen    row i is chosen iff it is uncommitted and
            (h_choose(i) * n_uncommitted) >> 32 < 20, h_choose = word 0 of
            (0, i, gstep, SYN_CHOOSE).  A chosen row gets +30 at
            t_i = (h_target(i) * V) >> 32, h_target = word 0 of (0, i, gstep, SYN_TARGET).
  committed rows get +30 at their own id.
  The +30 is one float32 addition.

Pins: tests/test_oracle_decode.py checks the expected accept count (20 per step
until fewer than 20 remain, so about 13 steps per canvas) and that noise rows
stay far below the commit threshold at every temperature in [0.4, 1].
"""
import numpy as np

from . import native, philox

SPIKE = np.float32(30.0)
CHOOSE_PER_STEP = 20


def synth_logits(ids, committed, gstep, seed, table, vocab, rows=None):
    """Logits [len(rows), V] float32 for the canvas state (ids, committed) at global step gstep."""
    ids = np.asarray(ids, dtype=np.int64)
    committed = np.asarray(committed, dtype=np.uint8)
    n = ids.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    table = np.asarray(table, dtype=np.float32)
    n_unc = int(n - committed.sum())
    jj = np.arange(vocab, dtype=np.uint64)
    # the noise part from the C helper when it is available (same draws)
    out = native.synth_noise(table, len(rows), vocab, seed, gstep, rows)
    if out is None:
        out = np.empty((len(rows), vocab), dtype=np.float32)
        for r, i in enumerate(rows):
            h = philox.word(seed, philox.STREAM_SYN_NOISE, gstep, int(i), c0=jj >> np.uint64(2),
                            w=(jj & np.uint64(3)).astype(np.int64))
            out[r] = table[(h >> np.uint32(16)).astype(np.int64)]
    for r, i in enumerate(rows):
        if committed[i]:
            out[r, ids[i]] = np.float32(out[r, ids[i]] + SPIKE)
        else:
            hc = int(philox.word(seed, philox.STREAM_SYN_CHOOSE, gstep, int(i)))
            if (hc * n_unc) >> 32 < CHOOSE_PER_STEP:
                ht = philox.word(seed, philox.STREAM_SYN_TARGET, gstep, int(i))
                t = int(philox.range_id(ht, vocab))
                out[r, t] = np.float32(out[r, t] + SPIKE)
    return out
