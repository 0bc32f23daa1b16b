"""Seeded synthetic inputs for the five canvas-denoising workloads.

This module only draws inputs: it holds none of the method's arithmetic and is
the one piece shared by the GPU path's tests/bench and the CPU oracle.  No
trained weights or datasets are involved; every tensor is drawn from a numpy
PCG64 generator seeded by SeedSequence([workload_id, tag]) so each tensor can be
drawn alone, in any order.

Workloads (shapes from the pages' decode setting: a 256-token canvas, a 262k
vocabulary, a 4096-token committed history, a 1024-token answer):
  1 tiny        N=256, P=256, 8/8 heads, D=64, fp32 Q/K/V ~ N(0,1); V=4096, d=512;
                logits ~ N(0,3) per step; E ~ N(0,0.02); ids uniform; 0 committed;
                8 steps, tau 0.9, greedy, T=1.
  2 mid         N=256, P=1024, 16/8 heads, D=128, bf16 Q/K/V ~ N(0,1); V=32768,
                d=2048; logits ~ N(0,4) per step; 77 (=round(0.3*256)) positions
                pre-committed with their initial ids; 8 steps.
  3 full vocab  sampler only: V=262144, d=3072; logits N(0,2) plus 12 at one
                uniformly drawn id per row; E ~ N(0,0.02); 1 step.
  4 long ctx    attention as 2 with P=4096, then the sampler of 3 (same E), one step.
  5 decode run  P=4096 prefix, 4 canvases of 256; per canvas fresh Q/K/V;
                E is workload 3's E; logits come from the threshold-tuned
                synthetic generator fed by a 65536-entry N(0,1) table drawn here.
bf16 tensors are drawn in float32 and rounded to nearest-even bf16 values (held
as float32 numbers that are exactly representable in bf16).
"""
import numpy as np

CONFIGS = {
    1: dict(name="tiny", n=256, n_prefix=256, hq=8, hkv=8, head_dim=64, qkv="f32",
            vocab=4096, d_model=512, logits="normal", logit_std=3.0, steps=8,
            precommit=0, tau=0.9),
    2: dict(name="mid", n=256, n_prefix=1024, hq=16, hkv=8, head_dim=128, qkv="bf16",
            vocab=32768, d_model=2048, logits="normal", logit_std=4.0, steps=8,
            precommit=77, tau=0.9),
    3: dict(name="full_vocab_sampler", n=256, vocab=262144, d_model=3072,
            logits="peaked", logit_std=2.0, peak=12.0, steps=1, precommit=0, tau=0.9),
    4: dict(name="long_context_step", n=256, n_prefix=4096, hq=16, hkv=8, head_dim=128,
            qkv="bf16", vocab=262144, d_model=3072, logits="peaked", logit_std=2.0,
            peak=12.0, steps=1, precommit=0, tau=0.9),
    5: dict(name="decode_run", n=256, n_prefix=4096, hq=16, hkv=8, head_dim=128,
            qkv="bf16", vocab=262144, d_model=3072, blocks=4, tau=0.9, s_max=48,
            t_start=0.8, t_end=0.4, seed=5),
}

_TAGS = dict(q=1, k_prefix=2, v_prefix=3, k_canvas=4, v_canvas=5, emb=6, ids=7,
             precommit=8, logits=9, peak=10, table=11)


def rng_for(workload, tag, *extra):
    return np.random.default_rng(np.random.SeedSequence([int(workload), _TAGS[tag], *extra]))


def round_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000))
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def attention_inputs(workload, n_prefix=None, block=None, n=None, hq=None, hkv=None,
                     head_dim=None, qkv=None):
    """(q, k_prefix, v_prefix, k_canvas, v_canvas) as float32 arrays.

    Overrides allow the same recipe at other shapes (edge-case tests).  For the
    decode run, ``block`` selects a canvas's fresh Q/K/V (the prefix is shared).
    """
    c = CONFIGS[workload]
    n = c["n"] if n is None else n
    p = c["n_prefix"] if n_prefix is None else n_prefix
    hq = c["hq"] if hq is None else hq
    hkv = c["hkv"] if hkv is None else hkv
    dh = c["head_dim"] if head_dim is None else head_dim
    qkv = c["qkv"] if qkv is None else qkv
    extra = () if block is None else (1000 + int(block),)
    shape_tag = (n, p, hq, hkv, dh)
    q = normal(rng_for(workload, "q", *shape_tag, *extra), (n, hq, dh))
    kp = normal(rng_for(workload, "k_prefix", *shape_tag), (p, hkv, dh))
    vp = normal(rng_for(workload, "v_prefix", *shape_tag), (p, hkv, dh))
    kc = normal(rng_for(workload, "k_canvas", *shape_tag, *extra), (n, hkv, dh))
    vc = normal(rng_for(workload, "v_canvas", *shape_tag, *extra), (n, hkv, dh))
    if qkv == "bf16":
        q, kp, vp, kc, vc = (round_bf16(t) for t in (q, kp, vp, kc, vc))
    return q, kp, vp, kc, vc


def fp8_codes(x):
    """OCP FP8 E4M3 bytes of float32 values (torch's round-to-nearest-even
    conversion); input preparation only."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def attention_inputs_fp8(workload, **overrides):
    """The same Q/K/V draws as attention_inputs (float32 recipe), as E4M3 bytes."""
    overrides["qkv"] = "f32"
    return tuple(fp8_codes(t) for t in attention_inputs(workload, **overrides))


def embedding(workload, vocab=None, d_model=None):
    """E [V, d] float32 ~ N(0, 0.02).  Workloads 4 and 5 reuse workload 3's table."""
    if workload in (4, 5):
        workload = 3
    c = CONFIGS[workload]
    vocab = c["vocab"] if vocab is None else vocab
    d_model = c["d_model"] if d_model is None else d_model
    return normal(rng_for(workload, "emb", vocab, d_model), (vocab, d_model), 0.02)


def initial_canvas(workload, n=None, vocab=None):
    """(ids int32 [N], committed uint8 [N]); committed positions keep their initial ids."""
    c = CONFIGS[workload]
    n = c["n"] if n is None else n
    vocab = c["vocab"] if vocab is None else vocab
    ids = rng_for(workload, "ids", n, vocab).integers(0, vocab, size=n).astype(np.int32)
    mask = np.zeros(n, dtype=np.uint8)
    k = c.get("precommit", 0)
    if k:
        pos = rng_for(workload, "precommit", n).choice(n, size=k, replace=False)
        mask[pos] = 1
    return ids, mask


def step_logits(workload, step, n=None, vocab=None):
    """Logits [N, V] float32 for one step of workloads 1-4."""
    c = CONFIGS[workload]
    n = c["n"] if n is None else n
    vocab = c["vocab"] if vocab is None else vocab
    x = normal(rng_for(workload, "logits", step, n, vocab), (n, vocab), c["logit_std"])
    if c["logits"] == "peaked":
        peak = rng_for(workload, "peak", step, n, vocab).integers(0, vocab, size=n)
        x[np.arange(n), peak] += np.float32(c["peak"])
    return x


def synth_table(size=65536):
    """The N(0,1) float32 table the decode run's synthetic logit generator indexes."""
    return normal(rng_for(5, "table", size), (size,))
