"""One diffusion-sampler step over a canvas (oracle side; test infrastructure only).

What the pages fix
  * Sampling runs over the whole 256-token canvas in full precision with a
    262k vocabulary, and besides the softmax it computes the self-conditioning
    embedding product (DiffusionGemma Technical Report, section 6 "Sampling");
    the self-conditioning state z_t is computed from a previous forward pass
    (Technical Report, section 8, "Finetuning procedure", around Eq. 13).
  * Generation is uniform (multinomial) diffusion: the canvas starts uniformly
    random and non-accepted tokens are renoised uniformly at random (explainer
    "DiffusionGemma: Google's open diffusion LLM", sections quoting report 3.1-3.3;
    aiboss88 page, "Uniform State Diffusion").
  * Confident tokens are locked in, the rest re-noised (AlphaSignal page, "How
    text diffusion actually works", items 2-3).
  * At most 48 denoising steps; temperature falls linearly from 0.8 to 0.4
    (explainer, "Sampler settings that decide DiffusionGemma latency", Table 2).

Readings taken where the pages are silent (each also listed in the design notes):
  R1  commit rule: an uncommitted position commits when its confidence
      kappa >= tau (inclusive).  kappa is the temperature-T probability of the
      candidate id.
  R2  commits are persistent within the canvas: a committed position is never
      changed again (monotone mask).
  R3  re-noise draws uniformly over all V ids (the current id included), one
      draw per (seed, step, position).
  R4  temperature: T = t_start, or with the schedule flag
      T = t_start + (t_end - t_start) * (s / (s_max - 1)), s = step within the
      canvas, all in float32 in that order, no fused multiply-add.
  R5  self-conditioning uses softmax at T = 1 for every row, committed or not:
      z = softmax(l) @ E.
  R6  candidate: greedy argmax of the logits, or with the Gumbel flag
      argmax(l * (1/T) + g) with g from oracle.philox.  Ties go to the smallest id.
  R11 on the last allowed step (s + 1 >= s_max) every remaining defined
      position commits its candidate.  Parity unpinned (a spec choice).
  Undefined rows (a NaN, a +inf, or no finite logit) get kappa = NaN and z = NaN,
  never commit, and are re-noised like any other non-accepted position.

Precision: softmax, z and kappa are float64.  The two decisions that turn floats
into integers are taken in float32, the GPU's precision: the Gumbel-perturbed
scores are float32 (l * invT rounded, then + g rounded), and the commit test is
float32(kappa) >= float32(tau).

Pins (tests/test_oracle_sampler.py): scipy softmax/logsumexp; E = I gives z = p;
an all-ones E column gives sum(p) = 1; uniform logits give the column mean of E;
a dominant spike gives its E row; z is linear in E; two-logit closed form
p = sigmoid((a - b) / T); brute-force Gumbel-max frequencies; monotone-mask,
commit-only and all-spike / all-uniform invariants; resume identity.
"""
from dataclasses import dataclass, replace

import numpy as np

from . import native, philox

GUMBEL = 1
COMMIT_ONLY = 2
AUTO_ADVANCE = 4
T_SCHEDULE = 8


@dataclass(frozen=True)
class Ctrl:
    seed: int = 0
    gstep: int = 0
    s_in_block: int = 0
    s_max: int = 48
    flags: int = 0
    tau: float = 0.9
    t_start: float = 1.0
    t_end: float = 1.0

    def advanced(self):
        return replace(self, gstep=self.gstep + 1, s_in_block=self.s_in_block + 1)


def temperature(ctrl):
    """Temperature as float32, reading R4 (Table 2's linear schedule over the step budget)."""
    t0 = np.float32(ctrl.t_start)
    if (ctrl.flags & T_SCHEDULE) and ctrl.s_max > 1:
        span = np.float32(np.float32(ctrl.t_end) - t0)
        frac = np.float32(np.float32(ctrl.s_in_block) / np.float32(ctrl.s_max - 1))
        return np.float32(t0 + np.float32(span * frac))
    return t0


def softmax64(rows, temp=1.0):
    """Row softmax of rows / temp in float64 (max-shifted)."""
    x = np.asarray(rows, dtype=np.float64) / float(temp)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def undefined_rows(logits):
    l = np.asarray(logits)
    return np.isnan(l).any(axis=1) | ~np.isfinite(l.max(axis=1)) | np.isposinf(l).any(axis=1)


def candidates(logits, ctrl, temp, rows=None):
    """Candidate id per row (R6) and the float32 top-2 gap used by the parity rule.

    Greedy: argmax of the logits; the gap is in probability units of p_T.
    Gumbel: argmax of the float32 perturbed score; the gap is in score units.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    n, vocab = l32.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    cand = np.zeros(len(rows), dtype=np.int64)
    gap = np.zeros(len(rows), dtype=np.float64)
    inv_t = np.float32(np.float32(1.0) / np.float32(temp))
    # Gumbel scores for all requested rows at once from the C helper (same draws,
    # evaluated natively); None when no C compiler is available
    fast = native.gumbel_scores(l32[rows], inv_t, ctrl.seed, ctrl.gstep, rows) \
        if (ctrl.flags & GUMBEL) else None
    for out_i, i in enumerate(rows):
        row = l32[i]
        if ctrl.flags & GUMBEL:
            if fast is not None:
                score = fast[out_i]
            else:
                g = philox.gumbel_row(ctrl.seed, ctrl.gstep, int(i), vocab)
                score = ((row * inv_t).astype(np.float32) + g).astype(np.float32)
            c = int(np.argmax(score))
            top2 = np.partition(score.astype(np.float64), -2)[-2:]
            gap[out_i] = top2[1] - top2[0]
        else:
            c = int(np.argmax(row))
            p = softmax64(row[None, :], temp)[0]
            top2 = np.partition(p, -2)[-2:]
            gap[out_i] = top2[1] - top2[0]
        cand[out_i] = c
    return cand, gap


def selfcond(logits, emb, rows=None):
    """z = softmax(l) @ E in float64 (R5), optionally for a subset of rows."""
    l = np.asarray(logits)
    if rows is not None:
        l = l[np.asarray(rows)]
    p = softmax64(l)
    e64 = emb if (isinstance(emb, np.ndarray) and emb.dtype == np.float64) else np.asarray(emb, dtype=np.float64)
    return p @ e64


def sampler_step(logits, emb, ids, committed, ctrl, z_rows="all"):
    """One sampler step.  Returns a dict with the new state and the diagnostics.

    logits [N,V] float32; emb [V,d] float32 (or float64); ids [N] int; committed [N] 0/1.
    z_rows: "all", None (skip z), or an index array of rows whose z is computed.
    """
    l = np.asarray(logits, dtype=np.float32)
    n, vocab = l.shape
    ids = np.asarray(ids, dtype=np.int64).copy()
    committed = np.asarray(committed, dtype=np.uint8).copy()
    temp = temperature(ctrl)
    bad = undefined_rows(l)

    safe = np.where(bad[:, None], 0.0, l.astype(np.float64))
    cand, gap = candidates(np.where(bad[:, None], np.float32(0), l), ctrl, temp)
    p_t = softmax64(safe, float(temp))
    kappa = p_t[np.arange(n), cand]
    kappa = np.where(bad, np.nan, kappa)

    last_step = ctrl.s_in_block + 1 >= ctrl.s_max
    accept = (~bad) & (committed == 0) & (
        (kappa.astype(np.float32) >= np.float32(ctrl.tau)) | last_step)
    new_ids = ids.copy()
    new_mask = committed.copy()
    new_ids[accept] = cand[accept]
    new_mask[accept] = 1
    renoise = (committed == 0) & ~accept
    if not (ctrl.flags & COMMIT_ONLY):
        pos = np.nonzero(renoise)[0]
        if len(pos):
            new_ids[pos] = philox.renoise_ids(ctrl.seed, ctrl.gstep, pos, vocab)
    else:
        renoise[:] = False

    if z_rows is None:
        z = None
    elif isinstance(z_rows, str) and z_rows == "all":
        z = selfcond(safe, emb)
        z[bad] = np.nan
    else:
        rows = np.asarray(z_rows)
        z = selfcond(safe, emb, rows)
        z[bad[rows]] = np.nan

    out_ctrl = ctrl.advanced() if (ctrl.flags & AUTO_ADVANCE) else ctrl
    return dict(ids=new_ids, committed=new_mask, z=z, kappa=kappa, cand=cand, gap=gap,
                accepted=accept, renoised=renoise, undefined=bad,
                n_uncommitted=int(n - new_mask.sum()), ctrl=out_ctrl, temperature=temp)


def init_canvas(ctrl, n, vocab):
    """Start of a canvas: uniform ids from the INIT stream, nothing committed, step 0."""
    ids = philox.init_ids(ctrl.seed, ctrl.gstep, np.arange(n), vocab)
    return ids, np.zeros(n, dtype=np.uint8), replace(ctrl, s_in_block=0)
