"""Denoising-step throughput on one MI355X.

One step = the whole hot path on one synthetic canvas: bidirectional canvas
attention over a 4096-token committed prefix plus the 256-token canvas (16 query
/ 8 KV heads, head_dim 128, bf16), then the sampler over a 262144-token
vocabulary with d_model 3072 (full softmax, z = softmax(logits)·E, confidence
commit / re-noise), replayed as one captured HIP graph.  Inputs are resident in
HBM before timing starts.

Prints one JSON line: steps/s, the roofline of the dominant kernel (the
self-conditioning contraction, priced by the method's own bytes and flops) from
per-kernel HIP events, roofline blocks for the whole sampler and for canvas
attention, fractions against measured peaks (copy and matrix-core probes), the
decode run through one captured step graph per canvas, and the CPU oracle's rate
on the same workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, calibrated
# on a plain copy; valid only for the kernel sources they were taken from
COUNTERS = os.path.join(ROOT, "profiles", "long_context_step_counters.json")
# the source files each kernel family is built from: a kernel's recorded counters
# stay valid while these files are unchanged
_CSRC = "block_text_diffusion_amd/csrc/"
KERNEL_SOURCES = {
    "samp": [_CSRC + "sampler.hip", _CSRC + "dg_common.hpp"],
    "attn": [_CSRC + "attention.hip", _CSRC + "dg_common.hpp"],
}
BF16_PEAK_TFLOPS = 2516.6
FP8_PEAK_TFLOPS = 5000.0
FP6_PEAK_TFLOPS = 10100.0
FP32_MFMA_PEAK_TFLOPS = 157.3
SAMPLER_KERNELS = ("samp_stats", "samp_gemm", "samp_combine", "samp_finalize")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="eager steps timed kernel by kernel (default: as many as --steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-workloads", action="store_true",
                    help="also time the tiny, mid and full-vocabulary-sampler workloads on the GPU and "
                         "with the CPU oracle (context; not part of the headline line's value)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time one plain bf16 GEMM of the contraction's shape through torch")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="bytes each way of the plain copy probe (measured HBM peak, counter calibration)")
    ap.add_argument("--no-probes", action="store_true", help="skip the copy and matrix-core peak probes")
    ap.add_argument("--no-decode-run", action="store_true", help="skip the decode runs")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline step, its per-kernel timing, the attention timing and the probes "
                         "(for counter runs under a profiler); implies --no-cpu-baseline and --no-decode-run")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    a = parse()
    if a.headline_only:
        a.no_cpu_baseline = a.no_decode_run = True
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_text_diffusion_amd as dg
    import workloads

    assert torch.cuda.is_available(), "no GPU"
    dg.load()
    c = workloads.CONFIGS[4]
    n, p, hq, hkv, hd = c["n"], c["n_prefix"], c["hq"], c["hkv"], c["head_dim"]
    vocab, dm = c["vocab"], c["d_model"]

    log("generating inputs (long-context step workload)")
    q, kp, vp, kc, vc = workloads.attention_inputs(4)
    emb = workloads.embedding(4)
    logits = workloads.step_logits(4, 0)
    ids, mask = workloads.initial_canvas(4)
    bf = torch.bfloat16
    dev = lambda x, dt=None: (torch.from_numpy(x).to(dt) if dt else torch.from_numpy(x)).cuda()
    T = dict(q=dev(q, bf), kp=dev(kp, bf), vp=dev(vp, bf), kc=dev(kc, bf), vc=dev(vc, bf),
             logits=dev(logits), ids=dev(ids.astype(np.int32)), mask=dev(mask))
    # E is converted once to the split-bf16 layout the sampler streams (load time, not per step)
    emb_f32 = dev(emb)
    torch.cuda.synchronize()
    tp = time.perf_counter()
    T["emb"] = dg.dg_embedding_pack(emb_f32)
    torch.cuda.synchronize()
    pack_ms = (time.perf_counter() - tp) * 1e3
    T["emb_f32"] = emb_f32          # the top-k sampler gathers rows of the plain fp32 table
    T["attn"] = torch.empty((n, hq, hd), dtype=torch.float32, device="cuda")
    T["z"] = torch.empty((n, dm), dtype=torch.float32, device="cuda")
    T["kappa"] = torch.empty(n, dtype=torch.float32, device="cuda")
    T["nu"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    T["ctrl"] = dg.make_ctrl(seed=4, tau=0.9, flags=dg.DG_AUTO_ADVANCE)
    step_args = (T["q"], T["kp"], T["vp"], T["kc"], T["vc"], T["attn"], T["logits"], T["emb"],
                 T["ids"], T["mask"], T["z"], T["kappa"], T["nu"], T["ctrl"])
    ws = torch.empty(dg.dg_denoise_workspace_bytes(n, p, hq, hkv, hd, vocab, dm), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    # ---- graph replay: the headline ----
    graph = dg.StepGraph(*step_args, workspace=ws)
    for _ in range(a.warmup):
        graph.launch()
    torch.cuda.synchronize()
    log(f"timing {a.steps} graph replays")
    t0 = time.perf_counter()
    for _ in range(a.steps):
        graph.launch()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / a.steps
    steps_per_s = a.steps / elapsed
    # spread of single replays (events between replays on the launch stream), after the timed region
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    evs[0].record()
    for i in range(a.steps):
        graph.launch()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_replay = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps)])
    replay_ms = {"median": round(float(np.median(per_replay)), 4),
                 "p10": round(float(np.percentile(per_replay, 10)), 4),
                 "p90": round(float(np.percentile(per_replay, 90)), 4)}

    # ---- per-kernel durations (HIP events on the launch stream, eager calls,
    # as many steps as the timed region, right after it) ----
    profile_steps = a.profile_steps or a.steps
    dg.dg_profile_enable(True)
    dg.dg_profile_read()
    for _ in range(profile_steps):
        dg.dg_denoise_step(*step_args, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    prof = dg.dg_profile_read()
    dg.dg_profile_enable(False)
    per_kernel_us = {k: 1e3 * ms / cnt for k, (ms, cnt) in prof.items()}
    log("per-kernel us: " + ", ".join(f"{k}={v:.1f}" for k, v in per_kernel_us.items()))
    graph.close()

    # Algorithmic work of the dominant kernel per launch (one step): the method
    # reads the logits and E once and writes z, and does 2 N V d flops.  The
    # contraction runs one fp16 product and two fp6 correction products per
    # fp32-accurate one; at 412.3 GFLOP over 3.493 GB (118 flop/B) it is below
    # the fp16 ridge (2516.6 / 8 = 315 flop/B), so the bound is HBM bandwidth.
    gemm_us = per_kernel_us["samp_gemm"]
    flops_method = 2.0 * n * vocab * dm                         # softmax(l)·E
    flops_fp16, flops_fp6 = flops_method, 2.0 * flops_method    # the products the matrix cores execute
    # matrix-core time at the datasheet peaks (fp16 = bf16 rate, fp6 four times it)
    split_floor_us = (flops_fp16 / BF16_PEAK_TFLOPS + flops_fp6 / FP6_PEAK_TFLOPS) / 1e12 * 1e6
    bytes_method = 4.0 * (n * vocab + vocab * dm + n * dm)      # logits + E + z, each once
    gbs = bytes_method / (gemm_us * 1e-6) / 1e9
    roofline = {
        "kernel": "samp_gemm",
        "bound": "hbm",
        "achieved": round(gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic("samp_gemm"),
        "avg_us": round(gemm_us, 2),
        "algorithmic_bytes": bytes_method,
        "algorithmic_flops": flops_method,
        "arithmetic_intensity": round(flops_method / bytes_method, 1),
        "hbm_floor_us": round(bytes_method / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
        # the split-precision products (fp16 + two fp6) against the datasheet
        # matrix-core peaks: the time they need at peak over the time taken
        "split_mfma_floor_us": round(split_floor_us, 1),
        "split_mfma_frac": round(split_floor_us / gemm_us, 4),
        # from the committed rocprofv3 counter run of the same sources (None if
        # stale): the clock the chip held and the matrix cores' busy fraction
        "counters_clock_ghz": measured_counter("samp_gemm", "clock_ghz"),
        "counters_mfma_busy": measured_counter("samp_gemm", "mfma_busy"),
        "timing": "HIP events around each launch on its stream, eager steps right after the timed region",
    }
    # the whole sampler (four kernels) against the same HBM floor, and against
    # max(HBM floor, split-precision matrix-core floor)
    samp_us = sum(per_kernel_us[k] for k in SAMPLER_KERNELS if k in per_kernel_us)
    floor_hbm_us = bytes_method / (HBM_PEAK_GBS * 1e9) * 1e6
    floor_split_us = max(floor_hbm_us, split_floor_us)
    sampler = {"kernels": list(SAMPLER_KERNELS), "us": round(samp_us, 2),
               "bound": "hbm", "floor_us": round(floor_hbm_us, 1), "frac": round(floor_hbm_us / samp_us, 4),
               "floor_split_us": round(floor_split_us, 1), "frac_split": round(floor_split_us / samp_us, 4)}
    samp_traffic = [measured_traffic(k) for k in SAMPLER_KERNELS]
    if all(t is not None for t in samp_traffic):
        sampler["traffic"] = sum(samp_traffic)
        sampler["traffic_over_algorithmic"] = round(sum(samp_traffic) / bytes_method, 3)
    attn = bf16_attention_timing(torch, dg, T, n, p, hq, hkv, hd, a.steps)
    attn_traffic = [measured_traffic(k) for k in ("attn_partial", "attn_combine")]
    if all(t is not None for t in attn_traffic):
        attn["roofline"]["traffic"] = sum(attn_traffic)
        attn["roofline"]["traffic_over_algorithmic"] = round(sum(attn_traffic) / attn["roofline"]["algorithmic_bytes"],
                                                             3)
    attn["per_kernel_us_eager_events"] = {k: round(per_kernel_us[k], 2)
                                          for k in ("attn_partial", "attn_combine", "attn_fused")
                                          if k in per_kernel_us}
    log(f"roofline: samp_gemm {gemm_us:.1f} us = {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of HBM); "
        f"sampler {samp_us:.1f} us ({floor_hbm_us / samp_us:.3f}); attention {attn['us']:.2f} us "
        f"({attn['roofline']['frac']:.3f} of bf16 peak)")

    probes = None if a.no_probes else peak_probes(torch, dg, a.copy_probe_mib)
    if probes:
        roofline["secondary"] = {"measured_peak": probes["copy_gbs"], "unit": "GB/s",
                                 "frac": round(gbs / probes["copy_gbs"], 4),
                                 # the contraction's bytes are almost all reads
                                 "measured_read_peak": probes["read_gbs"],
                                 "frac_of_read": round(gbs / probes["read_gbs"], 4),
                                 # the probe measures bf16; fp16 runs at that rate, fp6 at four times it
                                 "split_mfma_frac": round((flops_fp16 + flops_fp6 / 4) / (gemm_us * 1e-6) / 1e12
                                                          / probes["mfma_tflops"], 4)}
        sampler["frac_measured_hbm"] = round(bytes_method / (probes["copy_gbs"] * 1e9) * 1e6 / samp_us, 4)
        attn["roofline"]["secondary"] = {"measured_peak": probes["mfma_tflops"], "unit": "TFLOP/s",
                                         "frac": round(attn["tflops"] / probes["mfma_tflops"], 4)}

    eb = batched = attn_fp8 = attn_batched = topk = None
    if not a.headline_only:
        # ---- the entropy-bounded sampler (the pages' default) on the same inputs ----
        eb = eb_sampler_timing(torch, dg, T, n, vocab, dm, a.steps)
        log(f"entropy-bounded sampler: {eb['ms_per_step']:.3f} ms per step")

        # ---- batches of canvases sharing one pass over E ----
        batched = batched_sampler_timing(torch, dg, T, n, vocab, dm, a.steps)
        log("batched sampler: " + ", ".join(f"B={r['batch']}: {r['ms_per_step']:.3f} ms "
                                            f"({r['canvas_steps_per_s']:.0f} canvas-steps/s)" for r in batched))

        # ---- FP8 (E4M3) attention on the same draws ----
        attn_fp8 = fp8_attention_timing(torch, dg, workloads, n, p, hq, hkv, hd, a.steps)
        log(f"fp8 attention: {attn_fp8['us']:.1f} us per call")

        # ---- a denoising pass and a KV-update pass batched in one launch ----
        attn_batched = batched_attention_timing(torch, dg, T, n, p, hq, hkv, hd, a.steps)
        log(f"batched attention (denoise + KV update): {attn_batched['us_batched']:.1f} us in one launch, "
            f"{attn_batched['us_two_calls']:.1f} us as two calls")

        # ---- the top-k truncated sampler (approximate), alone and after attention ----
        topk = topk_sampler_timing(torch, dg, T, n, p, hq, hkv, hd, vocab, dm, a.steps)
        log("top-k sampler: " + ", ".join(f"k={r['k']} B={r['batch']}: {r['sampler_ms']:.3f} ms"
                                          for r in topk["runs"]))

    # ---- the decode run: 4096-token prefix, four 256-token canvases, one step graph per canvas ----
    dec = dec_eb = None
    if not a.no_decode_run:
        dec = decode_run_timing(torch, dg, T["emb"], vocab, dm)
        log(f"decode run: {dec['tokens']} tokens in {dec['steps']} steps, {dec['tokens_per_s_wall']:.0f} tokens/s "
            f"wall, {dec['tokens_per_s_kernel']:.0f} tokens/s from step GPU time")
        dec_eb = decode_run_timing(torch, dg, T["emb"], vocab, dm, entropy_bounded=True)
        log(f"decode run, entropy-bounded: {dec_eb['tokens']} tokens in {dec_eb['steps']} steps, "
            f"{dec_eb['tokens_per_s_wall']:.0f} tokens/s wall")

    blas = None
    if a.blas_reference:
        # calibration only: one bf16 GEMM [N, V] x [V, d] (a third of the contraction's work)
        A = torch.randn(n, vocab, device="cuda").to(torch.bfloat16)
        B = (torch.randn(vocab, dm, device="cuda") * 0.02).to(torch.bfloat16)
        for _ in range(3):
            A @ B
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            A @ B
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / 10 * 1e6
        blas = {"us": round(us, 1), "tflops": round(2.0 * n * vocab * dm / (us * 1e-6) / 1e12, 1)}
        log(f"torch bf16 GEMM of the same shape: {us:.1f} us")
        del A, B

    cpu = oracle_block0 = None
    if not a.no_cpu_baseline:
        cpu, e64 = cpu_baseline(q, kp, vp, kc, vc, emb, logits, ids, mask)
        oracle_block0 = oracle_decode_block0(e64)
        del e64
    others = workload_sweep(torch, dg, workloads) if a.all_workloads else None

    out = {
        "metric": "denoise steps/s (attn+sampler) at 262k vocab, 4096 ctx",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # attention in bf16; the sampler's contraction in fp16 + fp6 products
        # with fp32 accumulation, its softmax statistics in fp32
        "dtype": "bf16+fp16+fp6+f32",
        "data": "synthetic",
        "config": {"workload": "long_context_step: canvas 256, prefix 4096, 16q/8kv heads, head_dim 128 "
                               "bf16; vocab 262144, d_model 3072 fp32; one captured graph per step",
                   "canvas_tokens_per_s": round(256 * steps_per_s, 1),
                   "replay_ms": replay_ms,
                   "per_kernel_us_eager_events": {k: round(v, 2) for k, v in per_kernel_us.items()},
                   "per_kernel_note": "HIP events around each kernel of eager steps on the launch stream; "
                                      "the event pairs add a few us to the short kernels, the graph replays "
                                      "run them back to back (rocprofv3 in-graph durations in profiles/)",
                   "sampler": sampler,
                   "peak_probes": probes,
                   "embedding_pack_ms_once": round(pack_ms, 2),
                   "attention": attn,
                   "other_workloads": others,
                   "eb_sampler": eb,
                   "decode_run": dec,
                   "decode_run_entropy_bounded": dec_eb,
                   "oracle_decode_block0": oracle_block0,
                   "batched_sampler": batched,
                   "topk_sampler": topk,
                   "attention_fp8": attn_fp8,
                   "attention_batched": attn_batched,
                   "blas_reference_bf16_gemm": blas},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def decode_run_timing(torch, dg, emb_packed, vocab, dm, entropy_bounded=False):
    """The decode-run workload on the device: a 4096-token prefix, then four
    256-token canvases.  Each canvas gets one captured step graph (canvas
    attention over the prefix as it stands, then the Gumbel sampler with T
    0.8 -> 0.4), captured before the timed region; the prefix grows by 256
    rows per canvas through the KV append.  Per step: the synthetic logits
    (eagerly, outside the graph: they stand in for the model), then one graph
    replay bracketed by two events, then one host read of the open count (or
    the stop flag).  Threshold mode runs until no position is open;
    entropy-bounded mode (the pages' default; the accepted positions stand in
    for the committed mask of the synthetic generator) until adaptive stopping
    fires or s_max steps.

    tokens_per_s_kernel follows Eq. 12 of the Technical Report: tokens per
    forward pass over the mean step GPU time (the graph replays, attention and
    sampler).  tokens_per_s_wall is the whole loop on the host clock, with the
    synthetic logits, canvas starts, host reads and KV appends."""
    import workloads
    c = workloads.CONFIGS[5]
    n, p0, hq, hkv, hd = c["n"], c["n_prefix"], c["hq"], c["hkv"], c["head_dim"]
    bf = torch.bfloat16
    dev = lambda x, dt=None: (torch.from_numpy(x).to(dt) if dt else torch.from_numpy(x)).cuda()
    _, kp, vp, _, _ = workloads.attention_inputs(5, block=0)
    total = p0 + c["blocks"] * n
    kbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    vbuf = torch.empty((total, hkv, hd), dtype=bf, device="cuda")
    kbuf[:p0] = dev(kp, bf)
    vbuf[:p0] = dev(vp, bf)
    blocks = []
    for b in range(c["blocks"]):
        q, _, _, kc, vc = workloads.attention_inputs(5, block=b)
        blocks.append((dev(q, bf), dev(kc, bf), dev(vc, bf)))
    table = dev(workloads.synth_table())
    logits = torch.empty((n, vocab), dtype=torch.float32, device="cuda")
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    mask = torch.zeros(n, dtype=torch.uint8, device="cuda")
    z = torch.empty((n, dm), dtype=torch.float32, device="cuda")
    kappa = torch.empty(n, dtype=torch.float32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ent = torch.empty(n, dtype=torch.float32, device="cuda")
    amax = torch.empty(n, dtype=torch.int32, device="cuda")
    status = torch.zeros(16, dtype=torch.uint8, device="cuda")
    attn = torch.empty((n, hq, hd), dtype=torch.float32, device="cuda")
    ctrl = dg.make_ctrl(seed=c["seed"], s_max=c["s_max"], tau=c["tau"], t_start=c["t_start"],
                        t_end=c["t_end"], flags=dg.DG_AUTO_ADVANCE | dg.DG_GUMBEL | dg.DG_T_SCHEDULE)
    ws = torch.empty(dg.dg_denoise_workspace_bytes(n, total - n, hq, hkv, hd, vocab, dm), dtype=torch.uint8,
                     device="cuda")
    # one step graph per canvas, each over the prefix length that canvas sees
    graphs = []
    for b, (q, kc, vc) in enumerate(blocks):
        p = p0 + b * n
        if entropy_bounded:
            graphs.append(dg.StepGraphEB(q, kbuf[:p], vbuf[:p], kc, vc, attn, logits, emb_packed, ids, mask, z,
                                         ent, amax, status, ctrl, workspace=ws))
        else:
            graphs.append(dg.StepGraph(q, kbuf[:p], vbuf[:p], kc, vc, attn, logits, emb_packed, ids, mask, z,
                                       kappa, nu, ctrl, workspace=ws))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(c["blocks"] * c["s_max"])]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps, p = 0, p0
    per_block = []
    for b, (q, kc, vc) in enumerate(blocks):
        dg.dg_canvas_init(ids, mask, ctrl, vocab)
        if entropy_bounded:
            amax.fill_(-1)
        s_block = 0
        for _ in range(c["s_max"]):
            dg.dg_synth_logits(logits, ids, mask, ctrl, table)
            evs[steps][0].record()
            graphs[b].launch()
            evs[steps][1].record()
            steps += 1
            s_block += 1
            if entropy_bounded:
                if dg.read_eb_status(status)["stop"]:
                    break
            elif int(nu.item()) == 0:
                break
        dg.dg_kv_append(kbuf, vbuf, kc, vc, p)
        p += n
        per_block.append(s_block)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = np.array([evs[k][0].elapsed_time(evs[k][1]) for k in range(steps)])
    for g in graphs:
        g.close()
    tokens = c["blocks"] * n
    tpf = tokens / steps                        # tokens per forward pass
    t_fwd_ms = float(step_ms.mean())
    return {"tokens": tokens, "steps": steps, "steps_per_canvas": per_block, "tokens_per_forward": round(tpf, 2),
            "seconds_wall": round(dt, 5), "tokens_per_s_wall": round(tokens / dt, 1),
            "step_gpu_ms_mean": round(t_fwd_ms, 4), "step_gpu_ms_median": round(float(np.median(step_ms)), 4),
            "tokens_per_s_kernel": round(tpf / (t_fwd_ms * 1e-3), 1),
            "note": "one captured step graph (attention + sampler) per canvas, prefix 4096 + 256 b; synthetic "
                    "logits written on the device before each replay (outside the step GPU time); one host read "
                    "per step" + ("; entropy-bounded sampler, budget 0.1, adaptive stop at mean entropy 0.005"
                                  if entropy_bounded else "")}


def batched_sampler_timing(torch, dg, T, n, vocab, dm, steps, batches=(2, 4, 8)):
    """The threshold sampler over B canvases in one pass (each canvas its own
    control block): ms per batched step and canvas-steps/s.  The step's logits
    are replicated B times; greedy candidates, T = 1."""
    out = []
    for B in batches:
        logits = T["logits"].repeat(B, 1)
        ids = T["ids"].repeat(B)
        mask = torch.zeros(B * n, dtype=torch.uint8, device="cuda")
        z = torch.empty((B * n, dm), dtype=torch.float32, device="cuda")
        nu = torch.zeros(B, dtype=torch.int32, device="cuda")
        ctrl = dg.stack_ctrl([dg.make_ctrl(seed=10 + b, tau=0.9, flags=dg.DG_AUTO_ADVANCE) for b in range(B)])
        ws = torch.empty(dg.dg_sampler_workspace_bytes_batched(n, B, vocab, dm), dtype=torch.uint8, device="cuda")
        run = lambda: dg.dg_sampler_step_batched(logits, T["emb"], ids, mask, z, None, nu, ctrl, B, workspace=ws)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        k = max(5, steps // B)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / k
        out.append({"batch": B, "ms_per_step": round(ms, 4), "canvas_steps_per_s": round(B * 1e3 / ms, 1)})
        del logits, ids, mask, z, ws
        torch.cuda.empty_cache()
    return out


def bf16_attention_timing(torch, dg, T, n, p, hq, hkv, hd, steps, n_sets=16):
    """Canvas attention of the headline step alone (bf16 inputs, the long-context
    shapes): eager calls back to back between two events on the launch stream,
    cycling through n_sets copies of Q/K/V (16 x 17.8 MB of K/V, more than the
    256 MB last-level cache) so no call finds its K/V left in cache by the
    previous one.  Per-kernel HIP events around each launch add a few
    microseconds of event overhead to kernels this short, so the attention
    figure is taken this way."""
    ws = torch.empty(dg.dg_attention_workspace_bytes(n, p, hq, hkv, hd), dtype=torch.uint8, device="cuda")
    sets = [tuple(T[k].clone() for k in ("q", "kp", "vp", "kc", "vc")) for _ in range(n_sets)]
    run = lambda i: dg.dg_canvas_attention(*sets[i % n_sets], out=T["attn"], workspace=ws)
    for i in range(n_sets):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # algorithmic work per call: QK^T and PV over the 4352 keys for 256 x 16
    # query rows; bytes: Q, prefix and canvas K/V once (bf16), O (fp32)
    flops = 4.0 * n * (p + n) * hd * hq
    nbytes = 2.0 * n * hq * hd + 2.0 * 2.0 * (p + n) * hkv * hd + 4.0 * n * hq * hd
    tflops = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "tflops": round(tflops, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
                         "algorithmic_bytes": nbytes, "arithmetic_intensity": round(flops / nbytes, 1),
                         "floor_us": round(flops / (BF16_PEAK_TFLOPS * 1e12) * 1e6, 2)},
            "timing": f"eager calls back to back between two events (every kernel of a call), "
                      f"{n_sets} rotated Q/K/V sets"}


def peak_probes(torch, dg, copy_mib):
    """Measured peaks on this machine: a plain copy (bytes read + written per
    second), a plain read, and the matrix-core loop probe (bf16 flops per
    second), each timed with events over several launches after a warm-up."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src = torch.ones(copy_mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dg.dg_probe_copy(dst, src)
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        dg.dg_probe_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    copy_gbs = 2.0 * (copy_mib << 20) / (copy_ms * 1e-3) / 1e9
    del dst
    # a plain read of 4x the copy's buffer (more than the 256 MB last-level cache)
    big = torch.empty(4 * (copy_mib << 18), dtype=torch.float32, device="cuda")
    big.fill_(1.0)
    sink = dg.dg_probe_read(big)
    for _ in range(2):
        dg.dg_probe_read(big, sink)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dg.dg_probe_read(big, sink)
    e1.record()
    torch.cuda.synchronize()
    read_ms = e0.elapsed_time(e1) / reps
    read_gbs = 4.0 * (copy_mib << 20) / (read_ms * 1e-3) / 1e9
    del src, big, sink
    for _ in range(2):
        dg.dg_probe_mfma_bf16()
    torch.cuda.synchronize()
    e0.record()
    flops = 0.0
    for _ in range(reps):
        flops += dg.dg_probe_mfma_bf16()
    e1.record()
    torch.cuda.synchronize()
    mfma_tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    log(f"probes: copy {copy_gbs:.0f} GB/s, read {read_gbs:.0f} GB/s, matrix cores {mfma_tflops:.0f} TFLOP/s (bf16)")
    return {"copy_gbs": round(copy_gbs, 1), "copy_mib_each_way": copy_mib, "copy_ms": round(copy_ms, 4),
            "read_gbs": round(read_gbs, 1), "read_mib": 4 * copy_mib, "read_ms": round(read_ms, 4),
            "mfma_tflops": round(mfma_tflops, 1),
            "mfma_probe": "1024 workgroups x 4 waves x 2048 iterations x 4 independent 32x32x16 bf16 MFMA chains"}


def batched_attention_timing(torch, dg, T, n, p, hq, hkv, hd, steps, n_sets=8):
    """A denoising pass (bidirectional) and a KV-update pass (causal) of two
    long-context sequences: one batched launch against the same two passes as
    two calls.  The calls cycle through n_sets copies (8 x 35.7 MB of K/V, more
    than the 256 MB last-level cache).  Both passes are counted at the full key
    length, since the kernel computes every block of the causal canvas too."""
    two = lambda x: torch.stack([x, x]).contiguous()
    sets = [tuple(two(T[k]) for k in ("q", "kp", "vp", "kc", "vc")) for _ in range(n_sets)]
    out = torch.empty((2, n, hq, hd), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dg.dg_attention_batched_workspace_bytes(2, n, p, hq, hkv, hd),
                         dg.dg_attention_workspace_bytes(n, p, hq, hkv, hd)), dtype=torch.uint8, device="cuda")

    def batched(i):
        dg.dg_canvas_attention_batched(*sets[i % n_sets], [p, p], [False, True], out=out, workspace=ws)

    def separate(i):
        q, kp, vp, kc, vc = sets[i % n_sets]
        dg.dg_canvas_attention(q[0], kp[0], vp[0], kc[0], vc[0], out=out[0], workspace=ws)
        dg.dg_canvas_attention(q[1], kp[1], vp[1], kc[1], vc[1], out=out[1], workspace=ws, causal=True)

    res = {}
    for name, run in (("batched", batched), ("two_calls", separate)):
        for i in range(n_sets):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / steps
    flops = 2 * 4.0 * n * (p + n) * hd * hq
    return {"us_batched": round(res["batched"], 2), "us_two_calls": round(res["two_calls"], 2),
            "tflops_batched": round(flops / (res["batched"] * 1e-6) / 1e12, 1),
            "frac_bf16_peak_batched": round(flops / (res["batched"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "sequences": "2 x (canvas 256, prefix 4096): one bidirectional, one causal"}


def fp8_attention_timing(torch, dg, workloads, n, p, hq, hkv, hd, steps, n_sets=32):
    """Canvas attention with OCP E4M3 inputs (the long-context shapes), eager
    calls between two events, and the per-kernel split.  The calls cycle
    through n_sets copies of Q/K/V (32 x 8.9 MB of K/V, more than the 256 MB
    last-level cache)."""
    base = [torch.from_numpy(x).cuda() for x in workloads.attention_inputs_fp8(4)]
    sets = [tuple(t.clone() for t in base) for _ in range(n_sets)]
    out = torch.empty((n, hq, hd), dtype=torch.float32, device="cuda")
    ws = torch.empty(dg.dg_attention_workspace_bytes(n, p, hq, hkv, hd), dtype=torch.uint8, device="cuda")
    run = lambda i: dg.dg_canvas_attention_fp8(*sets[i % n_sets], 1.0, 1.0, 1.0, out=out, workspace=ws)
    for i in range(n_sets):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    dg.dg_profile_enable(True)
    dg.dg_profile_read()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    prof = dg.dg_profile_read()
    dg.dg_profile_enable(False)
    flops = 4.0 * n * (p + n) * hd * hq
    kv_bytes = 2.0 * (p + n) * hkv * hd          # K and V, one byte per element
    tflops = flops / (us * 1e-6) / 1e12
    # half the flops (Q.K^T) run on the FP8 matrix cores, half (P.V) on bf16:
    # the floor is (F/2)/fp8 peak + (F/2)/bf16 peak
    mixed_peak = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / BF16_PEAK_TFLOPS)
    return {"us": round(us, 2), "tflops": round(tflops, 1),
            "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
            "frac_mixed_peak": round(tflops / mixed_peak, 4), "mixed_peak_tflops": round(mixed_peak, 1),
            "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "kv_mb": round(kv_bytes / 1e6, 2),
            "per_kernel_us": {k: round(1e3 * t / c, 2) for k, (t, c) in prof.items()},
            "note": "E4M3 Q/K/V; Q.K^T on the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4), V staged exactly "
                    "as bf16 and P.V on bf16; fp32 softmax"}


def topk_sampler_timing(torch, dg, T, n, p, hq, hkv, hd, vocab, dm, steps, ks=(64, 256), batches=(1, 8)):
    """The top-k truncated threshold sampler on the step's logits (replicated
    over B canvases): ms per sampler step, per-kernel averages at B = 1, the HBM
    rate of its algorithmic bytes (logits once, the gathered E rows, z), and
    at B = 1 a whole step (attention over the 4352 keys, then this sampler)
    timed eagerly between two events."""
    runs = []
    attn_ws = torch.empty(dg.dg_attention_workspace_bytes(n, p, hq, hkv, hd), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k in ks:
        for B in batches:
            logits = T["logits"] if B == 1 else T["logits"].repeat(B, 1)
            ids = T["ids"].repeat(B)
            mask = torch.zeros(B * n, dtype=torch.uint8, device="cuda")
            z = torch.empty((B * n, dm), dtype=torch.float32, device="cuda")
            kappa = torch.empty(B * n, dtype=torch.float32, device="cuda")
            nu = torch.zeros(B, dtype=torch.int32, device="cuda")
            ctrl = dg.stack_ctrl([dg.make_ctrl(seed=20 + b, tau=0.9, flags=dg.DG_AUTO_ADVANCE) for b in range(B)])
            ws = torch.empty(dg.dg_sampler_workspace_bytes_topk(n, B, vocab, dm, k), dtype=torch.uint8,
                             device="cuda")
            run = lambda: dg.dg_sampler_step_topk(logits, T["emb_f32"], ids, mask, z, kappa, nu, ctrl, k, batch=B,
                                                  workspace=ws)
            for _ in range(3):
                run()
            torch.cuda.synchronize()
            reps = max(10, steps // B)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            nbytes = 4.0 * B * (n * vocab + n * k * dm + n * dm)
            rec = {"k": k, "batch": B, "sampler_ms": round(ms, 4), "canvas_steps_per_s": round(B * 1e3 / ms, 1),
                   "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if B == 1:
                dg.dg_profile_enable(True)
                dg.dg_profile_read()
                for _ in range(reps):
                    run()
                torch.cuda.synchronize()
                prof = dg.dg_profile_read()
                dg.dg_profile_enable(False)
                rec["per_kernel_us"] = {kk: round(1e3 * t / c, 2) for kk, (t, c) in prof.items()}
                step = lambda: (dg.dg_canvas_attention(T["q"], T["kp"], T["vp"], T["kc"], T["vc"], T["attn"],
                                                       workspace=attn_ws), run())
                for _ in range(3):
                    step()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    step()
                e1.record()
                torch.cuda.synchronize()
                sms = e0.elapsed_time(e1) / reps
                rec["step_ms_with_attention"] = round(sms, 4)
                rec["steps_per_s_with_attention"] = round(1e3 / sms, 1)
            runs.append(rec)
            del ws, z, kappa
    torch.cuda.empty_cache()
    return {"note": "approximate sampler: per row only the k largest logits are kept (ties to the smaller id); "
                    "z gathers k rows of the fp32 table; greedy, T = 1", "runs": runs}


def eb_sampler_timing(torch, dg, T, n, vocab, dm, steps):
    """Time the entropy-bounded sampler step (sampler only, no attention) on the
    step's logits: eager steps between two events, then per-kernel averages."""
    acc = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ent = torch.empty(n, dtype=torch.float32, device="cuda")
    amax = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    status = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ids = T["ids"].clone()
    ctrl = dg.make_ctrl(seed=4, s_max=1 << 30, flags=dg.DG_AUTO_ADVANCE | dg.DG_GUMBEL | dg.DG_T_SCHEDULE,
                        t_start=0.8, t_end=0.4)
    ws = torch.empty(dg.dg_sampler_workspace_bytes(n, vocab, dm), dtype=torch.uint8, device="cuda")
    run = lambda: dg.dg_sampler_step_eb(T["logits"], T["emb"], ids, acc, T["z"], ent, amax, status, ctrl,
                                        workspace=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    dg.dg_profile_enable(True)
    dg.dg_profile_read()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    prof = dg.dg_profile_read()
    dg.dg_profile_enable(False)
    return {"ms_per_step": round(ms, 4), "flags": "gumbel, T 0.8->0.4, budget 0.1",
            "per_kernel_us": {k: round(1e3 * t / c, 2) for k, (t, c) in prof.items()}}


def sources_sha256(kernel):
    """SHA-256 of the concatenated source files the kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.split("_")[0]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counter(kernel, field):
    """One field of the committed counter summary for a kernel (HBM bytes per
    launch, effective clock, matrix-core busy fraction), or None if the
    kernel's sources changed since its counters were taken."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
        k = rec["kernels"][kernel]
    except (OSError, ValueError, KeyError):
        return None
    if k.get("sources_sha256") != sources_sha256(kernel):
        return None
    return k.get(field)


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary (None if stale)."""
    return measured_counter(kernel, "hbm_bytes")


def workload_sweep(torch, dg, workloads):
    """GPU step time beside the CPU oracle's for the tiny (1), mid (2) and
    full-vocabulary sampler (3) workloads.  GPU: eager steps (attention then
    sampler; sampler only for 3) between two events, over the workload's own
    per-step logits.  Oracle: the same steps in fp64 numpy, z for all rows."""
    from oracle import sampler as S
    from oracle.attention import canvas_attention
    res = []
    for w in (1, 2, 3):
        c = workloads.CONFIGS[w]
        n, vocab, dm, nsteps = c["n"], c["vocab"], c["d_model"], c["steps"]
        log(f"workload {w} ({c['name']}): gpu")
        emb = workloads.embedding(w)
        logits = [workloads.step_logits(w, s) for s in range(nsteps)]
        ids, mask = workloads.initial_canvas(w)
        emb_t = torch.from_numpy(emb).cuda()
        pk = dg.dg_embedding_pack(emb_t)
        del emb_t
        lg = [torch.from_numpy(x).cuda() for x in logits]
        ids_t = torch.from_numpy(ids.astype(np.int32)).cuda()
        mask_t = torch.from_numpy(mask).cuda()
        z = torch.empty((n, dm), dtype=torch.float32, device="cuda")
        kappa = torch.empty(n, dtype=torch.float32, device="cuda")
        nu = torch.zeros(1, dtype=torch.int32, device="cuda")
        ctrl = dg.make_ctrl(seed=w, tau=c["tau"], flags=dg.DG_AUTO_ADVANCE)
        if w != 3:
            q, kp, vp, kc, vc = workloads.attention_inputs(w)
            dt = torch.bfloat16 if c["qkv"] == "bf16" else torch.float32
            A = [torch.from_numpy(x).to(dt).cuda() for x in (q, kp, vp, kc, vc)]
            attn = torch.empty((n, c["hq"], c["head_dim"]), dtype=torch.float32, device="cuda")
            ws = torch.empty(dg.dg_denoise_workspace_bytes(n, c["n_prefix"], c["hq"], c["hkv"], c["head_dim"],
                                                           vocab, dm), dtype=torch.uint8, device="cuda")
            step = lambda s: dg.dg_denoise_step(*A, attn, lg[s % nsteps], pk, ids_t, mask_t, z, kappa, nu, ctrl,
                                                workspace=ws)
        else:
            ws = torch.empty(dg.dg_sampler_workspace_bytes(n, vocab, dm), dtype=torch.uint8, device="cuda")
            step = lambda s: dg.dg_sampler_step(lg[0], pk, ids_t, mask_t, z, kappa, nu, ctrl, workspace=ws)
        reps = 40
        for s in range(4):
            step(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(reps):
            step(s)
        e1.record()
        torch.cuda.synchronize()
        gpu_ms = e0.elapsed_time(e1) / reps
        del lg, pk
        log(f"workload {w} ({c['name']}): oracle")
        e64 = emb.astype(np.float64)
        octrl = S.Ctrl(seed=w, tau=c["tau"], flags=S.AUTO_ADVANCE)
        o_steps = nsteps if w != 3 else 1
        t0 = time.perf_counter()
        for s in range(o_steps):
            if w != 3:
                canvas_attention(q, kp, vp, kc, vc)
            S.sampler_step(logits[s], e64, ids, mask, octrl, z_rows="all")
        cpu_ms = (time.perf_counter() - t0) * 1e3 / o_steps
        res.append({"workload": w, "name": c["name"], "gpu_ms_per_step": round(gpu_ms, 4),
                    "gpu_steps_per_s": round(1e3 / gpu_ms, 1), "oracle_ms_per_step": round(cpu_ms, 1),
                    "oracle_steps": o_steps, "what": "attention + sampler" if w != 3 else "sampler only"})
        log(f"workload {w}: gpu {gpu_ms:.3f} ms, oracle {cpu_ms:.0f} ms per step")
    return res


def host_cpu():
    """The host's CPU: cores this process may run on, the core count, and the model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": usable, "cpu_count": os.cpu_count(), "model": model}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def cpu_baseline(q, kp, vp, kc, vc, emb, logits, ids, mask):
    """The CPU oracle on the same workload: one full step (attention + sampler,
    z for all rows).  Returns the record and E widened to fp64 (reused)."""
    from oracle import sampler as S
    from oracle.attention import canvas_attention
    log("cpu baseline: widening E to fp64 (untimed input preparation)")
    e64 = emb.astype(np.float64)
    ctrl = S.Ctrl(seed=4, tau=0.9, flags=S.AUTO_ADVANCE)
    log("cpu baseline: timing oracle steps for at least 10 s")
    steps = 0
    t0 = time.perf_counter()
    while True:
        canvas_attention(q, kp, vp, kc, vc)
        S.sampler_step(logits, e64, ids, mask, ctrl, z_rows="all")
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or steps >= 30:
            break
    hc = host_cpu()
    return {"value": round(steps / dt, 4), "unit": "steps/s", "cores": int(blas_threads()), "kind": "oracle",
            "nproc": hc["nproc"], "cpu_model": hc["model"],
            "sample": f"{steps} full steps of the same workload (attention over 4352 keys for 256x16 query "
                      f"rows + sampler over 256x262144 logits with z for all rows) in {dt:.1f} s, "
                      f"fp64 numpy with {blas_threads()} BLAS threads; E widened to fp64 before timing"}, e64


def oracle_decode_block0(e64):
    """The oracle on the decode run's first canvas (prefix 4096): attention once
    (its Q/K/V are fixed for the canvas), then synthetic logits and a sampler
    step with z for all rows until the canvas is committed."""
    import workloads
    from oracle import decode, sampler as S
    c = workloads.CONFIGS[5]
    q, kp, vp, kc, vc = workloads.attention_inputs(5, block=0)
    ctrl = S.Ctrl(seed=c["seed"], s_max=c["s_max"], flags=S.AUTO_ADVANCE | S.GUMBEL | S.T_SCHEDULE,
                  tau=c["tau"], t_start=c["t_start"], t_end=c["t_end"])
    log("oracle: decode run, first canvas")
    t0 = time.perf_counter()
    recs, _ = decode.decode_run(kp, vp, [dict(q=q, k_canvas=kc, v_canvas=vc)], e64, workloads.synth_table(),
                                c["vocab"], ctrl, z_rows="all", max_blocks=1)
    dt = time.perf_counter() - t0
    steps = len(recs[0]["steps"])
    return {"seconds": round(dt, 2), "steps": steps, "tokens": c["n"], "tokens_per_s": round(c["n"] / dt, 2),
            "ms_per_step": round(dt * 1e3 / steps, 1), "cores": int(blas_threads()),
            "what": "attention once + per step synthetic logits and a sampler step with z for all 256 rows"}


if __name__ == "__main__":
    main()
