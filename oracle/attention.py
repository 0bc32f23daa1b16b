"""Bidirectional canvas attention (oracle side; test infrastructure only).

What the pages fix: during a denoising step every canvas token attends to the
committed history held in the KV cache and to all canvas tokens, with no causal
mask (DiffusionGemma Technical Report, section 6 "Attention" and section 9.1;
explainer "DiffusionGemma: Google's open diffusion LLM", section
"Block-autoregressive generation, one canvas after another", quoting report
section 3.1).  The pages give neither a scale, a soft-cap nor the head grouping;
the reading taken is standard scaled dot-product attention with scale 1/sqrt(D),
no soft-cap, rotary embedding already applied to the inputs, and grouped-query
heads where query head h reads KV head h // (Hq / Hkv).

Definition computed (float64 throughout, inputs widened exactly):
    K = [K_prefix ; K_canvas],  V = [V_prefix ; V_canvas]     (keys j = 0 .. P+N-1)
    O[i, h] = sum_j softmax_j(scale * q[i, h] . K[j, h // G]) * V[j, h // G]

The KV-update pass (the committed canvas written into the cache) is causal
over the canvas instead (explainer, "Block-autoregressive generation, one canvas
after another": a causal encoder reads the history).  Reading taken for the
causal flag: canvas row i attends to every prefix key and to canvas keys
0 .. i.

A batch of sequences (Technical Report part 4/6, paragraph "Eliminating
CPU-GPU synchronization": denoising passes and KV-update passes, with different
masks, can share one batch; explainer "DiffusionGemma: Google's open diffusion
LLM", section "Reference implementations in Transformers and vLLM": a
per-sequence causal flag).  Sequence s is the single-sequence definition
applied to its own inputs: prefix rows 0 .. n_prefix[s]-1 of its padded slab,
its canvas rows, and its own causal flag; padding rows are not keys.

Pins (tests/test_oracle_attention.py): explicit-loop brute force on tiny shapes;
torch's CPU scaled_dot_product_attention with repeated KV heads; closed forms
(one key gives v; scale 0 gives the mean of V; constant V gives that constant);
invariance under a permutation applied to canvas (or prefix) keys and values;
for a batch, torch's CPU scaled_dot_product_attention over the padded layout
with a boolean mask that hides each sequence's padding (and, where its flag is
set, the canvas keys after each row), and the outputs of one sequence unchanged
when another sequence's inputs or its own padding change.
"""
import numpy as np


def canvas_attention(q, k_prefix, v_prefix, k_canvas, v_canvas, scale=None, causal=False):
    """q [N,Hq,D]; k/v_prefix [P,Hkv,D] (P may be 0); k/v_canvas [N,Hkv,D] -> O [N,Hq,D] float64.

    causal: canvas row i sees the prefix and canvas keys 0..i only."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_canvas, dtype=np.float64)
    vc = np.asarray(v_canvas, dtype=np.float64)
    n, hq, d = q.shape
    hkv = kc.shape[1]
    if k_prefix is None or np.asarray(k_prefix).shape[0] == 0:
        keys, vals = kc, vc
    else:
        keys = np.concatenate([np.asarray(k_prefix, dtype=np.float64), kc], axis=0)
        vals = np.concatenate([np.asarray(v_prefix, dtype=np.float64), vc], axis=0)
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((n, hq, d), dtype=np.float64)
    p = keys.shape[0] - n
    masked = None
    if causal:
        j = np.arange(n)
        masked = j[None, :] > j[:, None]                       # canvas key j after row i
    for h in range(hq):
        kvh = h // group
        s = scale * (q[:, h, :] @ keys[:, kvh, :].T)          # [N, L]
        if masked is not None:
            s[:, p:][masked] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ vals[:, kvh, :]
    return out


def canvas_attention_batched(q, k_prefix, v_prefix, k_canvas, v_canvas, n_prefix, causal=None, scale=None):
    """q [B,N,Hq,D]; k/v_prefix [B,S,Hkv,D] (S = prefix stride, may be 0 or None);
    k/v_canvas [B,N,Hkv,D]; n_prefix: B lengths in [0, S]; causal: B flags or None
    -> O [B,N,Hq,D] float64.  Sequence s uses prefix rows 0..n_prefix[s]-1 only."""
    batch = np.asarray(q).shape[0]
    out = []
    for s in range(batch):
        np_s = int(n_prefix[s])
        kp = None if k_prefix is None else np.asarray(k_prefix)[s, :np_s]
        vp = None if v_prefix is None else np.asarray(v_prefix)[s, :np_s]
        flag = bool(causal[s]) if causal is not None else False
        out.append(canvas_attention(np.asarray(q)[s], kp, vp, np.asarray(k_canvas)[s],
                                    np.asarray(v_canvas)[s], scale=scale, causal=flag))
    return np.stack(out)
