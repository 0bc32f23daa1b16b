"""Top-k truncation of the sampler step (oracle side; test infrastructure only:
nothing outside tests/, the smoke check and the CPU baseline imports it).

What the pages say: the authors expect truncating the sampling step to the
top k tokens to raise throughput at larger batch sizes with a negligible
effect on output quality (explainer "DiffusionGemma: Google's open diffusion
LLM", section "Throughput flips at about 32 concurrent users", which cites the
report's section 6 and Figure 12).  Nothing more is given: no k, no rule for
ties and no statement of which quantities of the step are truncated.

Readings taken (each also listed in the design notes, K1-K4):
  K1  per row the kept set S holds the k largest logits, ties going to the
      smaller id (order: value descending, then id ascending).  Every other
      logit becomes -inf, and every quantity of the step (p, p_T, z, the
      candidate, kappa, the entropy) is then that of the truncated row, computed
      exactly as in the untruncated oracle.  k >= V leaves the row unchanged.
  K2  the truncation acts on the logits, so S does not depend on the
      temperature (T > 0 keeps the order), and the Gumbel candidate is drawn
      within S.
  K3  undefined rows (a NaN, a +inf, or no finite logit) are left unchanged, so
      they stay undefined.
  K4  when a row has fewer than k finite logits, the -inf entries that fill S
      carry weight 0.

Pins (tests/test_oracle_topk.py): brute force on tiny rows (an id is kept iff
fewer than k ids precede it in the order); torch.topk on rows of distinct
values; the renormalisation closed form p_k = p / sum over S of p (scipy
softmax of the full row); k = 1 gives a one-hot p, z = the E row of the
argmax and kappa = 1; equal logits keep the first k ids with p = 1/k and
entropy ln k; k >= V reproduces the untruncated step; Gumbel-max frequencies
within S follow the truncated p_T.
"""
import numpy as np

from . import eb as EB
from . import sampler as S


def keep_mask(row, k):
    """Boolean mask of the kept set of one row (reading K1)."""
    row = np.asarray(row)
    v = row.shape[0]
    if k >= v:
        return np.ones(v, dtype=bool)
    order = np.lexsort((np.arange(v), -row.astype(np.float64)))   # value desc, id asc
    mask = np.zeros(v, dtype=bool)
    mask[order[:k]] = True
    return mask


def truncate_top_k(logits, k):
    """Logits with everything outside each row's kept set set to -inf; undefined
    rows unchanged (K3).  Same dtype as the input."""
    l = np.array(logits, copy=True)
    bad = S.undefined_rows(l.astype(np.float32))
    for i in range(l.shape[0]):
        if not bad[i]:
            l[i, ~keep_mask(l[i], k)] = -np.inf
    return l


def sampler_step_topk(logits, emb, ids, committed, ctrl, k, z_rows="all"):
    """The threshold sampler step on the truncated logits."""
    return S.sampler_step(truncate_top_k(np.asarray(logits, np.float32), k), emb, ids, committed, ctrl,
                          z_rows=z_rows)


def eb_step_topk(logits, emb, ids, ctrl, k, prev_argmax=None, budget=EB.BUDGET,
                 stop_entropy=EB.STOP_ENTROPY, z_rows="all"):
    """The entropy-bounded step on the truncated logits."""
    return EB.eb_step(truncate_top_k(np.asarray(logits, np.float32), k), emb, ids, ctrl, prev_argmax, budget,
                      stop_entropy, z_rows=z_rows)
