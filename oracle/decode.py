"""Block-autoregressive decode loop (oracle side; test infrastructure only).

The model denoises one 256-token canvas until it is finished, commits it to the
history, stores it in the KV cache and starts the next canvas (explainer
"DiffusionGemma: Google's open diffusion LLM", section "Block-autoregressive
generation, one canvas after another", quoting report section 3.1; AlphaSignal
page, "How text diffusion actually works", item 4).  Without a model between
attention and sampler, each canvas's Q/K/V are inputs fixed for the canvas and
the logits come from oracle.synth.

Per canvas:
  ids <- INIT draws, mask <- 0, s_in_block <- 0
  repeat: logits <- synth(state); one sampler step (auto-advance)
  until no position is uncommitted (the forced final commit of reading R11
  bounds this at s_max steps)
  append the canvas K/V rows to the prefix.
"""
from dataclasses import replace

import numpy as np

from . import attention, sampler, synth


def decode_run(prefix_k, prefix_v, blocks, emb, table, vocab, ctrl, z_rows=None,
               with_attention=True, max_blocks=None):
    """Run the canvases in ``blocks`` (dicts with q, k_canvas, v_canvas).

    Returns a list of per-canvas records: attention output, the per-step
    sampler results (ids, mask, kappa, candidates, gaps) and the final ids.
    """
    ctrl = replace(ctrl, flags=ctrl.flags | sampler.AUTO_ADVANCE)
    kp = np.asarray(prefix_k, dtype=np.float64)
    vp = np.asarray(prefix_v, dtype=np.float64)
    records = []
    for b, blk in enumerate(blocks):
        if max_blocks is not None and b >= max_blocks:
            break
        n = blk["k_canvas"].shape[0]
        ids, mask, ctrl = sampler.init_canvas(ctrl, n, vocab)
        rec = dict(block=b, init_ids=ids.copy(), n_prefix=kp.shape[0], steps=[])
        if with_attention:
            rec["attention"] = attention.canvas_attention(
                blk["q"], kp, vp, blk["k_canvas"], blk["v_canvas"])
        while True:
            logits = synth.synth_logits(ids, mask, ctrl.gstep, ctrl.seed, table, vocab)
            res = sampler.sampler_step(logits, emb, ids, mask, ctrl, z_rows=z_rows)
            rec["steps"].append(dict(gstep=ctrl.gstep, s_in_block=ctrl.s_in_block,
                                     ids=res["ids"], committed=res["committed"],
                                     kappa=res["kappa"], cand=res["cand"], gap=res["gap"],
                                     z=res["z"], n_uncommitted=res["n_uncommitted"]))
            ids, mask, ctrl = res["ids"], res["committed"], res["ctrl"]
            if res["n_uncommitted"] == 0:
                break
        rec["final_ids"] = ids
        records.append(rec)
        kp = np.concatenate([kp, np.asarray(blk["k_canvas"], dtype=np.float64)], axis=0)
        vp = np.concatenate([vp, np.asarray(blk["v_canvas"], dtype=np.float64)], axis=0)
    return records, ctrl
