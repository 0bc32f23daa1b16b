"""MI355X (gfx950) canvas-denoising kernels for block text diffusion: Python binding.

Thin marshalling layer over the C ABI in libdg.so (include/dg.h).  Functions
carry the C names and take torch tensors that already live on the GPU; torch is
used only for device memory and the current stream.  Every computation runs in
the library's HIP kernels.
"""
import ctypes

from . import _lib
from ._lib import (DG_ATTN_CAUSAL, DG_AUTO_ADVANCE, DG_BF16, DG_COMMIT_ONLY, DG_F32, DG_FP8_E4M3, DG_GUMBEL,
                   DG_T_SCHEDULE, DgCtrl, DgError, check, load)

__all__ = [
    "dg_canvas_attention", "dg_canvas_attention_noalloc", "dg_static_scratch_bytes", "dg_canvas_attention_batched", "dg_attention_batched_workspace_bytes",
    "dg_canvas_attention_fp8", "dg_sampler_step", "dg_sampler_step_f32", "dg_sampler_step_eb", "read_eb_status",
    "dg_sampler_step_batched", "dg_sampler_step_eb_batched", "dg_sampler_workspace_bytes_batched",
    "dg_sampler_step_topk", "dg_sampler_step_eb_topk", "dg_sampler_workspace_bytes_topk",
    "stack_ctrl", "dg_embedding_pack", "dg_embedding_packed_bytes", "dg_denoise_step", "dg_denoise_step_eb", "dg_denoise_step_fp8", "StepGraph", "StepGraphEB",
    "StepGraphFP8", "dg_canvas_init",
    "dg_kv_append", "dg_synth_logits", "dg_philox_fill", "dg_attention_workspace_bytes",
    "dg_sampler_workspace_bytes", "dg_denoise_workspace_bytes", "dg_profile_enable",
    "dg_profile_read", "dg_probe_mfma_bf16", "dg_probe_copy", "dg_probe_read", "make_ctrl", "read_ctrl", "write_ctrl", "DG_GUMBEL", "DG_COMMIT_ONLY",
    "DG_AUTO_ADVANCE", "DG_T_SCHEDULE", "DG_ATTN_CAUSAL", "DG_F32", "DG_BF16", "DG_FP8_E4M3", "DgError", "load",
]


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtypes, device=True):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} dtype {t.dtype} not in {dtypes}")
    return t


def _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, out, batched=False):
    """Cross-tensor checks the C ABI cannot make from raw pointers: one dtype for
    Q/K/V, matching head counts, head_dim and canvas length, and the shape and
    dtype of a caller-supplied output.  Returns (n, hq, hkv, d, prefix rows)."""
    torch = _torch()
    lead = 1 if batched else 0
    if q.dim() != 3 + lead or k_canvas.dim() != 3 + lead or v_canvas.dim() != 3 + lead:
        raise ValueError("attention: q, k_canvas, v_canvas must be [%sn, heads, d]" % ("batch, " if batched else ""))
    b = q.shape[0] if batched else 1
    n, hq, d = q.shape[lead:]
    hkv = k_canvas.shape[lead + 1]
    tensors = [q, k_canvas, v_canvas]
    if tuple(k_canvas.shape) != tuple(v_canvas.shape) or tuple(k_canvas.shape[lead:]) != (n, hkv, d) \
            or (batched and k_canvas.shape[0] != b):
        raise ValueError(f"attention: canvas K/V shape {tuple(k_canvas.shape)} does not match q {tuple(q.shape)}")
    rows = 0
    if k_prefix is not None:
        if v_prefix is None or tuple(k_prefix.shape) != tuple(v_prefix.shape) or k_prefix.dim() != 3 + lead \
                or tuple(k_prefix.shape[lead + 1:]) != (hkv, d) or (batched and k_prefix.shape[0] != b):
            raise ValueError("attention: prefix K/V must both be [%sn_prefix, hkv, d]" % ("batch, " if batched else ""))
        rows = k_prefix.shape[lead]
        tensors += [k_prefix, v_prefix]
    if len({t.dtype for t in tensors}) != 1:
        raise ValueError("attention: q and every K/V tensor must share one dtype")
    if out is not None:
        want = (b, n, hq, d) if batched else (n, hq, d)
        if tuple(out.shape) != want or out.dtype != torch.float32 or not out.is_contiguous() \
                or out.device.type != "cuda":
            raise ValueError(f"attention: out must be a contiguous float32 GPU tensor of shape {want}")
    return n, hq, hkv, d, rows


def _qkv_dtype(t):
    torch = _torch()
    return DG_BF16 if t.dtype == torch.bfloat16 else DG_F32


def _workspace(nbytes, device, ws):
    torch = _torch()
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---- workspace queries ----
def dg_attention_workspace_bytes(n_canvas, n_prefix, hq, hkv, head_dim):
    return load().dg_attention_workspace_bytes(n_canvas, n_prefix, hq, hkv, head_dim)


def dg_sampler_workspace_bytes(n_canvas, vocab, d_model):
    return load().dg_sampler_workspace_bytes(n_canvas, vocab, d_model)


def dg_canvas_attention_fp8(q, k_prefix, v_prefix, k_canvas, v_canvas, q_scale=1.0, k_scale=1.0, v_scale=1.0,
                            out=None, scale=0.0, workspace=None, stream=None, causal=False):
    """Q/K/V as OCP FP8 E4M3 bytes (uint8 tensors, or torch.float8_e4m3fn) with
    per-tensor scales; output float32 [N, Hq, D]."""
    torch = _torch()
    dt = (torch.uint8, torch.float8_e4m3fn)
    _need(q, "q", dt); _need(k_canvas, "k_canvas", dt); _need(v_canvas, "v_canvas", dt)
    if k_prefix is not None and k_prefix.shape[0]:
        _need(k_prefix, "k_prefix", dt); _need(v_prefix, "v_prefix", dt)
    n, hq, hkv, d, n_prefix = _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, out)
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    ws = _workspace(dg_attention_workspace_bytes(n, n_prefix, hq, hkv, d), q.device, workspace)
    check(load().dg_canvas_attention_fp8(_ptr(q), _ptr(k_prefix) if n_prefix else None,
                                         _ptr(v_prefix) if n_prefix else None, _ptr(k_canvas), _ptr(v_canvas),
                                         _ptr(out), n, n_prefix, hq, hkv, d, float(scale), float(q_scale),
                                         float(k_scale), float(v_scale), DG_ATTN_CAUSAL if causal else 0,
                                         _ptr(ws), ws.numel(), _stream(stream)))
    return out


def dg_embedding_packed_bytes(vocab, d_model):
    return load().dg_embedding_packed_bytes(vocab, d_model)


def dg_embedding_pack(emb, packed=None, stream=None):
    """E [V, d] float32 on the GPU -> the fp16 + fp6 layout dg_sampler_step streams (uint8 tensor)."""
    torch = _torch()
    _need(emb, "emb", (torch.float32,))
    vocab, d = emb.shape
    if packed is None:
        packed = torch.empty(dg_embedding_packed_bytes(vocab, d), dtype=torch.uint8, device=emb.device)
    check(load().dg_embedding_pack(_ptr(emb), _ptr(packed), vocab, d, _stream(stream)))
    return packed


def dg_denoise_workspace_bytes(n_canvas, n_prefix, hq, hkv, head_dim, vocab, d_model):
    return load().dg_denoise_workspace_bytes(n_canvas, n_prefix, hq, hkv, head_dim, vocab, d_model)


# ---- control block ----
def make_ctrl(seed=0, gstep=0, s_in_block=0, s_max=48, flags=0, tau=0.9, t_start=1.0, t_end=1.0,
              device="cuda"):
    """A dg_ctrl in device memory (40-byte uint8 tensor)."""
    torch = _torch()
    c = DgCtrl(seed=seed, gstep=gstep, s_in_block=s_in_block, s_max=s_max, flags=flags, tau=tau,
               t_start=t_start, t_end=t_end, reserved=0)
    host = torch.frombuffer(bytearray(bytes(c)), dtype=torch.uint8)
    return host.to(device)


def write_ctrl(ctrl_t, **fields):
    cur = read_ctrl(ctrl_t)
    cur.update(fields)
    torch = _torch()
    c = DgCtrl(**cur)
    ctrl_t.copy_(torch.frombuffer(bytearray(bytes(c)), dtype=torch.uint8))


def read_ctrl(ctrl_t, index=0):
    raw = bytes(ctrl_t.cpu().numpy().tobytes()[40 * index:40 * index + 40])
    c = DgCtrl.from_buffer_copy(raw)
    return {f: getattr(c, f) for f, _ in DgCtrl._fields_}


# ---- the three calls of the denoising step ----
def dg_canvas_attention(q, k_prefix, v_prefix, k_canvas, v_canvas, out=None, scale=0.0,
                        workspace=None, stream=None, causal=False):
    torch = _torch()
    dt = (torch.bfloat16, torch.float32)
    _need(q, "q", dt); _need(k_canvas, "k_canvas", dt); _need(v_canvas, "v_canvas", dt)
    if k_prefix is not None and k_prefix.shape[0]:
        _need(k_prefix, "k_prefix", dt); _need(v_prefix, "v_prefix", dt)
    n, hq, hkv, d, n_prefix = _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, out)
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    nbytes = dg_attention_workspace_bytes(n, n_prefix, hq, hkv, d)
    ws = _workspace(nbytes, q.device, workspace)
    check(load().dg_canvas_attention_ex(_ptr(q), _ptr(k_prefix) if n_prefix else None,
                                        _ptr(v_prefix) if n_prefix else None, _ptr(k_canvas),
                                        _ptr(v_canvas), _ptr(out), n, n_prefix, hq, hkv, d,
                                        _qkv_dtype(q), float(scale), DG_ATTN_CAUSAL if causal else 0,
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def dg_static_scratch_bytes():
    return load().dg_static_scratch_bytes()


def dg_canvas_attention_noalloc(q, k_prefix, v_prefix, k_canvas, v_canvas, out, scale=0.0, stream=None,
                                causal=False):
    """dg_canvas_attention without a workspace: the library's static device
    scratch serves as workspace.  out [N, Hq, D] float32 is required (the call
    allocates nothing); calls that overlap in time on one GPU race."""
    torch = _torch()
    dt = (torch.bfloat16, torch.float32)
    _need(q, "q", dt); _need(k_canvas, "k_canvas", dt); _need(v_canvas, "v_canvas", dt)
    _need(out, "out", (torch.float32,))
    if k_prefix is not None and k_prefix.shape[0]:
        _need(k_prefix, "k_prefix", dt); _need(v_prefix, "v_prefix", dt)
    n, hq, hkv, d, n_prefix = _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, out)
    check(load().dg_canvas_attention_noalloc(_ptr(q), _ptr(k_prefix) if n_prefix else None,
                                             _ptr(v_prefix) if n_prefix else None, _ptr(k_canvas),
                                             _ptr(v_canvas), _ptr(out), n, n_prefix, hq, hkv, d, _qkv_dtype(q),
                                             float(scale), DG_ATTN_CAUSAL if causal else 0, _stream(stream)))
    return out


def dg_attention_batched_workspace_bytes(batch, n_canvas, prefix_stride, hq, hkv, head_dim):
    return load().dg_attention_batched_workspace_bytes(batch, n_canvas, prefix_stride, hq, hkv, head_dim)


def dg_canvas_attention_batched(q, k_prefix, v_prefix, k_canvas, v_canvas, n_prefix, causal=None, out=None,
                                scale=0.0, workspace=None, stream=None):
    """q [B, n, hq, d]; k_prefix / v_prefix [B, stride, hkv, d] or None (stride 0);
    k_canvas / v_canvas [B, n, hkv, d]; n_prefix and causal: B host values.
    Returns out [B, n, hq, d] float32."""
    torch = _torch()
    dt = (torch.bfloat16, torch.float32)
    _need(q, "q", dt); _need(k_canvas, "k_canvas", dt); _need(v_canvas, "v_canvas", dt)
    if k_prefix is not None and k_prefix.shape[1]:
        _need(k_prefix, "k_prefix", dt); _need(v_prefix, "v_prefix", dt)
    n, hq, hkv, d, stride = _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, out, batched=True)
    batch = q.shape[0]
    if len(n_prefix) != batch:
        raise ValueError(f"n_prefix has {len(n_prefix)} entries for a batch of {batch}")
    nps = (ctypes.c_int32 * batch)(*[int(x) for x in n_prefix])
    flags = None
    if causal is not None:
        if len(causal) != batch:
            raise ValueError(f"causal has {len(causal)} entries for a batch of {batch}")
        flags = (ctypes.c_uint8 * batch)(*[1 if c else 0 for c in causal])
    if out is None:
        out = torch.empty((batch, n, hq, d), dtype=torch.float32, device=q.device)
    nbytes = dg_attention_batched_workspace_bytes(batch, n, stride, hq, hkv, d)
    ws = _workspace(nbytes, q.device, workspace)
    check(load().dg_canvas_attention_batched(_ptr(q), _ptr(k_prefix) if stride else None,
                                             _ptr(v_prefix) if stride else None, _ptr(k_canvas),
                                             _ptr(v_canvas), _ptr(out), nps, flags, batch, n, stride, hq, hkv,
                                             d, _qkv_dtype(q), float(scale), _ptr(ws), ws.numel(),
                                             _stream(stream)))
    return out


def dg_sampler_step(logits, emb_packed, canvas_ids, committed, selfcond, confidence, n_uncommitted,
                    ctrl, workspace=None, stream=None):
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb_packed, "emb_packed", (torch.uint8,))
    _need(canvas_ids, "canvas_ids", (torch.int32,)); _need(committed, "committed", (torch.uint8,))
    _need(selfcond, "selfcond", (torch.float32,)); _need(n_uncommitted, "n_uncommitted", (torch.int32, torch.uint32))
    _need(ctrl, "ctrl", (torch.uint8,))
    if confidence is not None:
        _need(confidence, "confidence", (torch.float32,))
    n, vocab = logits.shape
    d = selfcond.shape[1]
    if emb_packed.numel() < dg_embedding_packed_bytes(vocab, d):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    nbytes = dg_sampler_workspace_bytes(n, vocab, d)
    ws = _workspace(nbytes, logits.device, workspace)
    check(load().dg_sampler_step(_ptr(logits), _ptr(emb_packed), _ptr(canvas_ids), _ptr(committed),
                                 _ptr(selfcond), _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl),
                                 n, vocab, d, _ptr(ws), ws.numel(), _stream(stream)))


def dg_sampler_step_f32(logits, emb, canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl,
                        workspace=None, stream=None):
    """dg_sampler_step on the plain float32 table E [V, d] (d a multiple of 4)."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb, "emb", (torch.float32,))
    _need(canvas_ids, "canvas_ids", (torch.int32,)); _need(committed, "committed", (torch.uint8,))
    _need(selfcond, "selfcond", (torch.float32,)); _need(n_uncommitted, "n_uncommitted", (torch.int32, torch.uint32))
    _need(ctrl, "ctrl", (torch.uint8,))
    if confidence is not None:
        _need(confidence, "confidence", (torch.float32,))
    n, vocab = logits.shape
    d = selfcond.shape[1]
    if tuple(emb.shape) != (vocab, d):
        raise ValueError("emb must be [vocab, d_model]")
    ws = _workspace(dg_sampler_workspace_bytes(n, vocab, d), logits.device, workspace)
    check(load().dg_sampler_step_f32(_ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(committed), _ptr(selfcond),
                                     _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl), n, vocab, d, _ptr(ws),
                                     ws.numel(), _stream(stream)))


def dg_sampler_step_eb(logits, emb_packed, canvas_ids, accepted, selfcond, entropy, argmax, status,
                       ctrl, budget=0.1, stop_entropy=0.005, workspace=None, stream=None):
    """Entropy-bounded sampler step.  status is a 16-byte uint8 device tensor
    (read it with read_eb_status); argmax is in/out (previous step's greedy ids)."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb_packed, "emb_packed", (torch.uint8,))
    _need(canvas_ids, "canvas_ids", (torch.int32,)); _need(accepted, "accepted", (torch.uint8,))
    _need(selfcond, "selfcond", (torch.float32,)); _need(argmax, "argmax", (torch.int32,))
    _need(status, "status", (torch.uint8,)); _need(ctrl, "ctrl", (torch.uint8,))
    if entropy is not None:
        _need(entropy, "entropy", (torch.float32,))
    if status.numel() < 16:
        raise ValueError("status needs 16 bytes")
    n, vocab = logits.shape
    d = selfcond.shape[1]
    if emb_packed.numel() < dg_embedding_packed_bytes(vocab, d):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    ws = _workspace(dg_sampler_workspace_bytes(n, vocab, d), logits.device, workspace)
    check(load().dg_sampler_step_eb(_ptr(logits), _ptr(emb_packed), _ptr(canvas_ids), _ptr(accepted),
                                    _ptr(selfcond), _ptr(entropy), _ptr(argmax), _ptr(status), _ptr(ctrl),
                                    float(budget), float(stop_entropy), n, vocab, d, _ptr(ws), ws.numel(),
                                    _stream(stream)))


def dg_sampler_workspace_bytes_batched(n_canvas, batch, vocab, d_model):
    return load().dg_sampler_workspace_bytes_batched(n_canvas, batch, vocab, d_model)


def stack_ctrl(ctrls):
    """Concatenate device control blocks (make_ctrl outputs) into one [batch * 40] tensor."""
    return _torch().cat(list(ctrls))


def dg_sampler_step_batched(logits, emb_packed, canvas_ids, committed, selfcond, confidence,
                            n_uncommitted, ctrl, batch, workspace=None, stream=None):
    """A batch of canvases stacked along the rows (logits [batch * n, V]); ctrl
    holds `batch` control blocks (stack_ctrl), n_uncommitted `batch` counts."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb_packed, "emb_packed", (torch.uint8,))
    _need(canvas_ids, "canvas_ids", (torch.int32,)); _need(committed, "committed", (torch.uint8,))
    _need(selfcond, "selfcond", (torch.float32,)); _need(n_uncommitted, "n_uncommitted", (torch.int32, torch.uint32))
    _need(ctrl, "ctrl", (torch.uint8,))
    rows, vocab = logits.shape
    if rows % batch or ctrl.numel() < 40 * batch or n_uncommitted.numel() < batch:
        raise ValueError("rows must split into `batch` canvases with a control block and a count each")
    n = rows // batch
    d = selfcond.shape[1]
    if emb_packed.numel() < dg_embedding_packed_bytes(vocab, d):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    ws = _workspace(dg_sampler_workspace_bytes_batched(n, batch, vocab, d), logits.device, workspace)
    check(load().dg_sampler_step_batched(_ptr(logits), _ptr(emb_packed), _ptr(canvas_ids), _ptr(committed),
                                         _ptr(selfcond), _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl),
                                         n, batch, vocab, d, _ptr(ws), ws.numel(), _stream(stream)))


def dg_sampler_step_eb_batched(logits, emb_packed, canvas_ids, accepted, selfcond, entropy, argmax,
                               status, ctrl, batch, budget=0.1, stop_entropy=0.005, workspace=None,
                               stream=None):
    """Entropy-bounded step over a batch; status holds `batch` 16-byte records."""
    torch = _torch()
    rows, vocab = logits.shape
    if rows % batch or ctrl.numel() < 40 * batch or status.numel() < 16 * batch:
        raise ValueError("rows must split into `batch` canvases with a control block and a status each")
    n = rows // batch
    d = selfcond.shape[1]
    ws = _workspace(dg_sampler_workspace_bytes_batched(n, batch, vocab, d), logits.device, workspace)
    check(load().dg_sampler_step_eb_batched(_ptr(logits), _ptr(emb_packed), _ptr(canvas_ids), _ptr(accepted),
                                            _ptr(selfcond), _ptr(entropy), _ptr(argmax), _ptr(status),
                                            _ptr(ctrl), float(budget), float(stop_entropy), n, batch, vocab,
                                            d, _ptr(ws), ws.numel(), _stream(stream)))


def dg_sampler_workspace_bytes_topk(n, batch, vocab, d_model, top_k):
    return load().dg_sampler_workspace_bytes_topk(n, batch, vocab, d_model, top_k)


def dg_sampler_step_topk(logits, emb, canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl,
                         top_k, batch=1, workspace=None, stream=None):
    """Top-k truncated threshold step over `batch` stacked canvases; emb is the
    plain fp32 table [V, d] (not the packed image)."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb, "emb", (torch.float32,))
    _need(canvas_ids, "canvas_ids", (torch.int32,)); _need(committed, "committed", (torch.uint8,))
    _need(selfcond, "selfcond", (torch.float32,)); _need(n_uncommitted, "n_uncommitted", (torch.int32, torch.uint32))
    _need(ctrl, "ctrl", (torch.uint8,))
    rows, vocab = logits.shape
    if rows % batch or ctrl.numel() < 40 * batch or n_uncommitted.numel() < batch:
        raise ValueError("rows must split into `batch` canvases with a control block and a count each")
    n = rows // batch
    d = selfcond.shape[1]
    if tuple(emb.shape) != (vocab, d):
        raise ValueError("emb must be [vocab, d_model]")
    ws = _workspace(dg_sampler_workspace_bytes_topk(n, batch, vocab, d, top_k), logits.device, workspace)
    check(load().dg_sampler_step_topk(_ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(committed),
                                      _ptr(selfcond), _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl),
                                      n, batch, vocab, d, top_k, _ptr(ws), ws.numel(), _stream(stream)))


def dg_sampler_step_eb_topk(logits, emb, canvas_ids, accepted, selfcond, entropy, argmax, status, ctrl,
                            top_k, batch=1, budget=0.1, stop_entropy=0.005, workspace=None, stream=None):
    """Top-k truncated entropy-bounded step; emb is the plain fp32 table [V, d]."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,)); _need(emb, "emb", (torch.float32,))
    rows, vocab = logits.shape
    if rows % batch or ctrl.numel() < 40 * batch or status.numel() < 16 * batch:
        raise ValueError("rows must split into `batch` canvases with a control block and a status each")
    n = rows // batch
    d = selfcond.shape[1]
    if tuple(emb.shape) != (vocab, d):
        raise ValueError("emb must be [vocab, d_model]")
    ws = _workspace(dg_sampler_workspace_bytes_topk(n, batch, vocab, d, top_k), logits.device, workspace)
    check(load().dg_sampler_step_eb_topk(_ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(accepted),
                                         _ptr(selfcond), _ptr(entropy), _ptr(argmax), _ptr(status), _ptr(ctrl),
                                         float(budget), float(stop_entropy), n, batch, vocab, d, top_k,
                                         _ptr(ws), ws.numel(), _stream(stream)))


def read_eb_status(status_t, index=0):
    from ._lib import DgEbStatus
    raw = bytes(status_t.cpu().numpy().tobytes()[16 * index:16 * index + 16])
    st = DgEbStatus.from_buffer_copy(raw)
    return {f: getattr(st, f) for f, _ in DgEbStatus._fields_}


def _denoise_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits, emb,
                  canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, ws):
    n, hq, d = q.shape
    hkv = k_canvas.shape[1]
    n_prefix = 0 if k_prefix is None else k_prefix.shape[0]
    vocab = logits.shape[1]
    dm = selfcond.shape[1]
    if emb.numel() < dg_embedding_packed_bytes(vocab, dm):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    return (_ptr(q), _ptr(k_prefix) if n_prefix else None, _ptr(v_prefix) if n_prefix else None,
            _ptr(k_canvas), _ptr(v_canvas), _ptr(attn_out), n_prefix, hq, hkv, d, _qkv_dtype(q),
            float(scale), _ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(committed), _ptr(selfcond),
            _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl), n, vocab, dm, _ptr(ws), ws.numel())


def dg_denoise_step(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed,
                    canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, scale=0.0,
                    workspace=None, stream=None):
    emb = emb_packed
    n, hq, d = q.shape
    nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                        k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
    ws = _workspace(nbytes, q.device, workspace)
    args = _denoise_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits, emb,
                         canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, ws)
    check(load().dg_denoise_step(*args, _stream(stream)))


def _denoise_eb_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits, emb, canvas_ids,
                     accepted, selfcond, entropy, argmax, status, ctrl, budget, stop_entropy, ws):
    n, hq, d = q.shape
    hkv = k_canvas.shape[1]
    n_prefix = 0 if k_prefix is None else k_prefix.shape[0]
    vocab = logits.shape[1]
    dm = selfcond.shape[1]
    if emb.numel() < dg_embedding_packed_bytes(vocab, dm):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    return (_ptr(q), _ptr(k_prefix) if n_prefix else None, _ptr(v_prefix) if n_prefix else None,
            _ptr(k_canvas), _ptr(v_canvas), _ptr(attn_out), n_prefix, hq, hkv, d, _qkv_dtype(q),
            float(scale), _ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(accepted), _ptr(selfcond),
            _ptr(entropy), _ptr(argmax), _ptr(status), _ptr(ctrl), float(budget), float(stop_entropy),
            n, vocab, dm, _ptr(ws), ws.numel())


def dg_denoise_step_eb(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                       accepted, selfcond, entropy, argmax, status, ctrl, budget=0.1, stop_entropy=0.005,
                       scale=0.0, workspace=None, stream=None):
    """Attention then the entropy-bounded sampler step (dg_sampler_step_eb)."""
    n, hq, d = q.shape
    nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                        k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
    ws = _workspace(nbytes, q.device, workspace)
    args = _denoise_eb_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits, emb_packed,
                            canvas_ids, accepted, selfcond, entropy, argmax, status, ctrl, budget, stop_entropy,
                            ws)
    check(load().dg_denoise_step_eb(*args, _stream(stream)))


def _denoise_fp8_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, q_scale, k_scale, v_scale,
                      logits, emb, canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, ws):
    torch = _torch()
    dt = (torch.uint8, torch.float8_e4m3fn)
    _need(q, "q", dt); _need(k_canvas, "k_canvas", dt); _need(v_canvas, "v_canvas", dt)
    if k_prefix is not None and k_prefix.shape[0]:
        _need(k_prefix, "k_prefix", dt); _need(v_prefix, "v_prefix", dt)
    n, hq, hkv, d, n_prefix = _check_attention_tensors(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out)
    vocab = logits.shape[1]
    dm = selfcond.shape[1]
    if emb.numel() < dg_embedding_packed_bytes(vocab, dm):
        raise ValueError("emb_packed is smaller than dg_embedding_packed_bytes(vocab, d_model)")
    return (_ptr(q), _ptr(k_prefix) if n_prefix else None, _ptr(v_prefix) if n_prefix else None,
            _ptr(k_canvas), _ptr(v_canvas), _ptr(attn_out), n_prefix, hq, hkv, d, float(scale), float(q_scale),
            float(k_scale), float(v_scale), _ptr(logits), _ptr(emb), _ptr(canvas_ids), _ptr(committed),
            _ptr(selfcond), _ptr(confidence), _ptr(n_uncommitted), _ptr(ctrl), n, vocab, dm, _ptr(ws), ws.numel())


def dg_denoise_step_fp8(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                        committed, selfcond, confidence, n_uncommitted, ctrl, q_scale=1.0, k_scale=1.0,
                        v_scale=1.0, scale=0.0, workspace=None, stream=None):
    """FP8 (E4M3) attention inputs with per-tensor scales, then the sampler step."""
    n, hq, d = q.shape
    nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                        k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
    ws = _workspace(nbytes, q.device, workspace)
    args = _denoise_fp8_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, q_scale, k_scale, v_scale,
                             logits, emb_packed, canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl,
                             ws)
    check(load().dg_denoise_step_fp8(*args, _stream(stream)))


class StepGraph:
    """dg_step_graph_create / _launch / _destroy: one captured denoising step.

    Keeps references to every tensor the graph reads or writes so they outlive it.
    """

    def __init__(self, q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed,
                 canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, scale=0.0,
                 workspace=None):
        emb = emb_packed
        n, hq, d = q.shape
        nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                            k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
        self.ws = _workspace(nbytes, q.device, workspace)
        self._keep = (q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb, canvas_ids,
                      committed, selfcond, confidence, n_uncommitted, ctrl)
        args = _denoise_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits, emb,
                             canvas_ids, committed, selfcond, confidence, n_uncommitted, ctrl, self.ws)
        handle = ctypes.c_void_p()
        check(load().dg_step_graph_create(*args, ctypes.byref(handle)))
        self.handle = handle

    def launch(self, stream=None):
        check(load().dg_step_graph_launch(self.handle, _stream(stream)))

    def close(self):
        if self.handle:
            load().dg_step_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepGraphEB(StepGraph):
    """dg_step_graph_create_eb: one captured step with the entropy-bounded sampler."""

    def __init__(self, q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                 accepted, selfcond, entropy, argmax, status, ctrl, budget=0.1, stop_entropy=0.005,
                 scale=0.0, workspace=None):
        n, hq, d = q.shape
        nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                            k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
        self.handle = None
        self.ws = _workspace(nbytes, q.device, workspace)
        self._keep = (q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                      accepted, selfcond, entropy, argmax, status, ctrl)
        args = _denoise_eb_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, logits,
                                emb_packed, canvas_ids, accepted, selfcond, entropy, argmax, status, ctrl,
                                budget, stop_entropy, self.ws)
        handle = ctypes.c_void_p()
        check(load().dg_step_graph_create_eb(*args, ctypes.byref(handle)))
        self.handle = handle


class StepGraphFP8(StepGraph):
    """dg_step_graph_create_fp8: one captured step with FP8 attention inputs."""

    def __init__(self, q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                 committed, selfcond, confidence, n_uncommitted, ctrl, q_scale=1.0, k_scale=1.0, v_scale=1.0,
                 scale=0.0, workspace=None):
        n, hq, d = q.shape
        nbytes = dg_denoise_workspace_bytes(n, 0 if k_prefix is None else k_prefix.shape[0], hq,
                                            k_canvas.shape[1], d, logits.shape[1], selfcond.shape[1])
        self.handle = None
        self.ws = _workspace(nbytes, q.device, workspace)
        self._keep = (q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, logits, emb_packed, canvas_ids,
                      committed, selfcond, confidence, n_uncommitted, ctrl)
        args = _denoise_fp8_args(q, k_prefix, v_prefix, k_canvas, v_canvas, attn_out, scale, q_scale, k_scale,
                                 v_scale, logits, emb_packed, canvas_ids, committed, selfcond, confidence,
                                 n_uncommitted, ctrl, self.ws)
        handle = ctypes.c_void_p()
        check(load().dg_step_graph_create_fp8(*args, ctypes.byref(handle)))
        self.handle = handle


# ---- block loop helpers ----
def dg_canvas_init(canvas_ids, committed, ctrl, vocab, stream=None):
    check(load().dg_canvas_init(_ptr(canvas_ids), _ptr(committed), _ptr(ctrl), canvas_ids.numel(),
                                int(vocab), _stream(stream)))


def dg_kv_append(k_prefix, v_prefix, k_canvas, v_canvas, n_prefix, stream=None):
    """Copy the canvas K/V [n, hkv, d] to rows n_prefix.. of the prefix buffers,
    whose first dimension is the capacity the library checks against."""
    torch = _torch()
    dt = (torch.bfloat16, torch.float32)
    for t, name in ((k_prefix, "k_prefix"), (v_prefix, "v_prefix"), (k_canvas, "k_canvas"), (v_canvas, "v_canvas")):
        _need(t, name, dt)
    n, hkv, d = k_canvas.shape
    cap = k_prefix.shape[0]
    if tuple(v_prefix.shape) != tuple(k_prefix.shape) or tuple(v_canvas.shape) != (n, hkv, d) \
            or tuple(k_prefix.shape[1:]) != (hkv, d):
        raise ValueError("kv_append: prefix buffers must be [capacity, hkv, d] and canvas K/V [n, hkv, d]")
    if len({k_prefix.dtype, v_prefix.dtype, k_canvas.dtype, v_canvas.dtype}) != 1:
        raise ValueError("kv_append: all four tensors must share one dtype")
    check(load().dg_kv_append(_ptr(k_prefix), _ptr(v_prefix), _ptr(k_canvas), _ptr(v_canvas),
                              int(n_prefix), int(cap), n, hkv, d, _qkv_dtype(k_canvas), _stream(stream)))


def dg_synth_logits(logits, canvas_ids, committed, ctrl, table, stream=None):
    n, vocab = logits.shape
    check(load().dg_synth_logits(_ptr(logits), _ptr(canvas_ids), _ptr(committed), _ptr(ctrl),
                                 _ptr(table), table.numel(), n, vocab, _stream(stream)))


def dg_philox_fill(out, seed, c1, c2, c3, stream=None):
    check(load().dg_philox_fill(_ptr(out), out.numel(), int(seed), int(c1), int(c2), int(c3),
                                _stream(stream)))


# ---- peak probes ----
def dg_probe_mfma_bf16(n_workgroups=1024, iters=2048, stream=None):
    """Launch the matrix-core probe; returns its flop count (time it with events)."""
    torch = _torch()
    sink = torch.empty(n_workgroups * 256, dtype=torch.float32, device="cuda")
    check(load().dg_probe_mfma_bf16(_ptr(sink), int(n_workgroups), int(iters), _stream(stream)))
    return float(n_workgroups) * 4 * iters * 4 * 32768


def dg_probe_copy(dst, src, stream=None):
    """Copy src to dst (same byte size, GPU tensors) with the plain copy probe."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("probe_copy: dst and src must have the same byte size")
    check(load().dg_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(), _stream(stream)))


PROBE_READ_SINK_WORDS = 16384


def dg_probe_read(src, sink=None, stream=None):
    """Read src (a GPU tensor, 16-byte aligned, byte size a multiple of 16) with
    the plain read probe; sink: int32 GPU tensor of PROBE_READ_SINK_WORDS (made
    here if not given)."""
    if sink is None:
        sink = _torch().empty(PROBE_READ_SINK_WORDS, dtype=_torch().int32, device="cuda")
    if sink.numel() * sink.element_size() < 4 * PROBE_READ_SINK_WORDS:
        raise ValueError("probe_read: sink must hold 16384 uint32 words")
    check(load().dg_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))
    return sink


# ---- profiling ----
def dg_profile_enable(on=True):
    check(load().dg_profile_enable(1 if on else 0))


def dg_profile_read(max_kernels=32):
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int * max_kernels)()
    k = load().dg_profile_read(names, ms, cnt, max_kernels)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k)}
