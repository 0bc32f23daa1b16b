"""The entropy-bounded sampler step and adaptive stopping (oracle side; test
infrastructure only).

What the pages fix (explainer "DiffusionGemma: Google's open diffusion LLM",
section "A diffusion language model refines 256 tokens in 12 steps", quoting
report sections 3.1-3.3; Table 2 under "Sampler settings that decide
DiffusionGemma latency"):
  * each step ranks the canvas positions by the entropy of their predictive
    distribution and accepts them from the lowest entropy upward until an
    entropy budget (0.1) is used up;
  * every other position is re-noised uniformly at random;
  * tokens of the open canvas stay editable (section "Tokens stay editable
    within a canvas, then freeze"), so a position accepted at one step is
    re-decided at the next;
  * the canvas stops early when the mean entropy over the canvas is below a
    threshold (0.005) and the most likely tokens of two consecutive steps are
    identical; at most 48 steps.

Readings taken where the pages are silent (each also listed in the design notes):
  E1  entropy is that of the temperature-T distribution p_T = softmax(l / T), in
      nats, with 0 log 0 = 0.
  E2  acceptance: sort the defined positions by (entropy, position) ascending;
      position k of that order is accepted iff the running sum of the first
      k + 1 entropies is <= budget (inclusive).  The first position of the
      order is always accepted, so a step accepts at least one token when any
      row is defined.
  E3  an accepted position takes its candidate (greedy argmax, or the Gumbel
      sample with the Gumbel flag, as in the threshold sampler); every other
      position, including previously accepted ones, gets a re-noise draw.
  E4  the mean entropy is over the defined rows; with no defined row it is NaN
      and the canvas does not stop.  "Most likely tokens" are the greedy argmax
      ids; with no previous step the stability test fails.
  E5  when the stop test holds, the canvas becomes those most likely ids (the
      stable prediction) and the canvas is finished.
  E6  on the last allowed step (s + 1 >= s_max) every defined position takes
      its candidate.  Parity unpinned (a spec choice, like the threshold
      sampler's forced final commit).
  Undefined rows (a NaN, a +inf, or no finite logit) have entropy NaN and are
  never accepted.

Precision: entropies, sums and z in float64; the candidate decision in float32
as in oracle.sampler.

Pins (tests/test_oracle_eb.py): scipy.stats.entropy; uniform rows give log V;
two-logit rows give the binary entropy of sigmoid((a - b) / T); hand-built
budget cases; the at-least-one rule; stop flag truth table; re-noise of
previously accepted positions.
"""
from dataclasses import replace

import numpy as np

from . import philox
from . import sampler as S

BUDGET = 0.1
STOP_ENTROPY = 0.005


def entropy64(logits, temp):
    """Entropy in nats of softmax(l / T) per row, float64 (0 log 0 = 0)."""
    x = np.asarray(logits, dtype=np.float64) / float(temp)
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    s = e.sum(axis=1, keepdims=True)
    p = e / s
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return -plogp.sum(axis=1)


def accept_order(entropy, budget=BUDGET):
    """Accepted mask (E2) plus the sorted order and running sums it came from."""
    h = np.asarray(entropy, dtype=np.float64)
    n = h.shape[0]
    defined = ~np.isnan(h)
    pos = np.nonzero(defined)[0]
    order = pos[np.lexsort((pos, h[pos]))]          # by entropy, then position
    csum = np.cumsum(h[order])
    acc = np.zeros(n, dtype=bool)
    take = csum <= budget
    if len(order):
        take[0] = True
    acc[order[take]] = True
    return acc, order, csum


def eb_step(logits, emb, ids, ctrl, prev_argmax=None, budget=BUDGET, stop_entropy=STOP_ENTROPY,
            z_rows="all"):
    """One entropy-bounded step.  Returns the new ids, the accepted mask, the
    entropies, the greedy argmax ids, the mean entropy, the stop flag, z and
    the diagnostics used by the comparison rules."""
    l = np.asarray(logits, dtype=np.float32)
    n, vocab = l.shape
    ids = np.asarray(ids, dtype=np.int64)
    temp = S.temperature(ctrl)
    bad = S.undefined_rows(l)
    safe = np.where(bad[:, None], 0.0, l.astype(np.float64))
    h = entropy64(safe, float(temp))
    h[bad] = np.nan
    cand, gap = S.candidates(np.where(bad[:, None], np.float32(0), l), ctrl, temp)
    argmax = np.argmax(np.where(bad[:, None], np.float32(0), l), axis=1).astype(np.int64)
    acc, order, csum = accept_order(h, budget)
    defined = ~bad
    if ctrl.s_in_block + 1 >= ctrl.s_max:
        acc = defined.copy()
    new_ids = philox.renoise_ids(ctrl.seed, ctrl.gstep, np.arange(n), vocab)
    new_ids[acc] = cand[acc]
    mean_h = float(h[defined].mean()) if defined.any() else float("nan")
    stable = prev_argmax is not None and bool(np.array_equal(np.asarray(prev_argmax), argmax))
    stop = bool(mean_h < stop_entropy) and stable
    if stop:
        new_ids = argmax.copy()
    if z_rows is None:
        z = None
    elif isinstance(z_rows, str) and z_rows == "all":
        z = S.selfcond(safe, emb)
        z[bad] = np.nan
    else:
        rows = np.asarray(z_rows)
        z = S.selfcond(safe, emb, rows)
        z[bad[rows]] = np.nan
    out_ctrl = ctrl.advanced() if (ctrl.flags & S.AUTO_ADVANCE) else ctrl
    return dict(ids=new_ids, accepted=acc.astype(np.uint8), entropy=h, argmax=argmax, cand=cand,
                gap=gap, mean_entropy=mean_h, stop=stop, n_accepted=int(acc.sum()), order=order,
                csum=csum, z=z, ctrl=out_ctrl, temperature=temp, undefined=bad)


def eb_canvas(step_logits, emb, ctrl, n, vocab, s_max=48, budget=BUDGET, stop_entropy=STOP_ENTROPY):
    """Denoise one canvas with the entropy-bounded sampler until it stops or
    s_max steps ran; step_logits(ids, ctrl) supplies each step's logits."""
    ids, _, ctrl = S.init_canvas(ctrl, n, vocab)
    ctrl = replace(ctrl, flags=ctrl.flags | S.AUTO_ADVANCE)
    prev = None
    steps = []
    for _ in range(s_max):
        r = eb_step(step_logits(ids, ctrl), emb, ids, ctrl, prev, budget, stop_entropy, z_rows=None)
        steps.append(r)
        ids, ctrl, prev = r["ids"], r["ctrl"], r["argmax"]
        if r["stop"]:
            break
    return ids, steps, ctrl
