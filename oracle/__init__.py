"""CPU oracle for the canvas-denoising step of block text diffusion.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct numpy
implementation (float64 unless a decision must be taken in float32) of what the
GPU path computes. Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library never calls,
links or imports anything here, and nothing here imports the HIP library.

Modules
-------
philox     Philox4x32-10 counter-based generator and the derived uniform / Gumbel /
           range draws (Salmon et al., SC'11).
attention  Bidirectional canvas attention over the committed KV prefix plus the
           canvas (DiffusionGemma Technical Report, section 6 "Attention").
sampler    One diffusion-sampler step: full-vocabulary softmax, the
           self-conditioning product softmax(logits)·E, confidence commit and
           uniform re-noise (Technical Report, section 6 "Sampling"; explainer
           "DiffusionGemma: Google's open diffusion LLM", sections 3.1-3.3 quotes).
synth      The synthetic, threshold-tuned logit generator for the decode run.
decode     The block-autoregressive decode loop with KV append.

Parity status per function (pinned / unpinned) is listed in each module header.
"""
