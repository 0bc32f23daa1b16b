"""The C ABI without a GPU: the library loads, exports what include/dg.h declares,
answers workspace queries, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from block_text_diffusion_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdg.so is not built (run python -m block_text_diffusion_amd.build)")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dg_canvas_attention", "dg_sampler_step", "dg_denoise_step",
                     "dg_step_graph_create", "dg_step_graph_launch", "dg_step_graph_destroy"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    from block_text_diffusion_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_workspace_queries(lib):
    a = lib.dg_attention_workspace_bytes(256, 4096, 16, 8, 128)
    assert a > 0 and a % 256 == 0
    s = lib.dg_sampler_workspace_bytes(256, 262144, 3072)
    # statistics partials plus the split-K partial sums of z
    assert s >= 256 * 3072 * 4 and s % 256 == 0
    d = lib.dg_denoise_workspace_bytes(256, 4096, 16, 8, 128, 262144, 3072)
    assert d == max(a, s)
    assert lib.dg_attention_workspace_bytes(257, 0, 8, 8, 64) == 0
    assert lib.dg_attention_workspace_bytes(16, 0, 6, 4, 64) == 0
    assert lib.dg_attention_workspace_bytes(16, 0, 8, 8, 96) == 0
    assert lib.dg_sampler_workspace_bytes(16, 1, 64) == 0
    assert lib.dg_sampler_workspace_bytes(0, 100, 64) == 0


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x10004)


def attn(lib, **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, kc=FAKE, vc=FAKE, out=FAKE, n=16, np=8, hq=8, hkv=4, d=64,
             dtype=1, scale=0.0, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.dg_canvas_attention(a["q"], a["kp"], a["vp"], a["kc"], a["vc"], a["out"], a["n"],
                                   a["np"], a["hq"], a["hkv"], a["d"], a["dtype"], a["scale"],
                                   a["ws"], a["wsb"], a["stream"])


def test_attention_argument_errors(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    assert attn(lib, q=None) == DG_EINVAL
    assert attn(lib, kp=None) == DG_EINVAL
    assert attn(lib, n=0) == DG_EINVAL
    assert attn(lib, n=257) == DG_EUNSUPPORTED
    assert attn(lib, hq=6) == DG_EINVAL
    assert attn(lib, d=96) == DG_EUNSUPPORTED
    assert attn(lib, dtype=7) == DG_EUNSUPPORTED
    assert attn(lib, q=MIS) == DG_EINVAL
    assert attn(lib, np=-1) == DG_EINVAL
    assert attn(lib, n=256, np=4096, hq=16, hkv=8, d=128, wsb=1024) == DG_EWORKSPACE
    assert b"workspace" in lib.dg_last_error()


def attn_batched(lib, nps=(8, 0, 5), causal=(0, 1, 0), **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, kc=FAKE, vc=FAKE, out=FAKE, batch=3 if nps is None else len(nps),
             n=16, stride=8, hq=8, hkv=4, d=64, dtype=1, scale=0.0, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    np_arr = None if nps is None else (ctypes.c_int32 * len(nps))(*nps)
    c_arr = None if causal is None else (ctypes.c_uint8 * len(causal))(*causal)
    return lib.dg_canvas_attention_batched(a["q"], a["kp"], a["vp"], a["kc"], a["vc"], a["out"], np_arr, c_arr,
                                           a["batch"], a["n"], a["stride"], a["hq"], a["hkv"], a["d"],
                                           a["dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


def test_batched_attention_workspace_and_errors(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_FP8_E4M3
    one = lib.dg_attention_workspace_bytes(256, 4096, 16, 8, 128)
    assert lib.dg_attention_batched_workspace_bytes(1, 256, 4096, 16, 8, 128) == one
    # more sequences: fewer key chunks each, partials for every sequence
    four = lib.dg_attention_batched_workspace_bytes(4, 256, 4096, 16, 8, 128)
    assert four > 0 and four % 256 == 0
    assert lib.dg_attention_batched_workspace_bytes(0, 16, 8, 8, 4, 64) == 0
    assert lib.dg_attention_batched_workspace_bytes(65, 16, 8, 8, 4, 64) == 0
    assert lib.dg_attention_batched_workspace_bytes(2, 16, -1, 8, 4, 64) == 0
    assert attn_batched(lib, nps=None) == DG_EINVAL
    assert attn_batched(lib, nps=(8, 9, 0), causal=(0, 0, 0)) == DG_EINVAL      # 9 > prefix stride 8
    assert b"n_prefix[1]" in lib.dg_last_error()
    assert attn_batched(lib, nps=(8, -1, 0)) == DG_EINVAL
    assert attn_batched(lib, causal=(0, 2, 0)) == DG_EINVAL
    assert attn_batched(lib, batch=0, nps=(), causal=()) == DG_EINVAL
    assert attn_batched(lib, batch=65, nps=(0,) * 65, causal=None) == DG_EUNSUPPORTED
    assert attn_batched(lib, dtype=DG_FP8_E4M3) == DG_EUNSUPPORTED
    assert attn_batched(lib, kp=None) == DG_EINVAL                                # stride > 0 needs a prefix
    assert attn_batched(lib, out=MIS) == DG_EINVAL
    assert attn_batched(lib, stride=-1) == DG_EINVAL
    assert attn_batched(lib, n=256, stride=4096, hq=16, hkv=8, d=128, wsb=1024) == DG_EWORKSPACE


def samp(lib, **kw):
    a = dict(l=FAKE, e=FAKE, ids=FAKE, c=FAKE, z=FAKE, conf=None, nu=FAKE, ctrl=FAKE, n=16,
             v=1000, d=64, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.dg_sampler_step(a["l"], a["e"], a["ids"], a["c"], a["z"], a["conf"], a["nu"],
                               a["ctrl"], a["n"], a["v"], a["d"], a["ws"], a["wsb"], a["stream"])


def test_sampler_argument_errors(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    assert samp(lib, l=None) == DG_EINVAL
    assert samp(lib, ctrl=None) == DG_EINVAL
    assert samp(lib, v=1) == DG_EINVAL
    assert samp(lib, d=0) == DG_EINVAL
    assert samp(lib, n=300) == DG_EUNSUPPORTED
    assert samp(lib, e=MIS) == DG_EINVAL
    assert samp(lib, wsb=16) == DG_EWORKSPACE


def test_helper_argument_errors(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED
    assert lib.dg_canvas_init(None, FAKE, FAKE, 16, 100, None) == DG_EINVAL
    assert lib.dg_canvas_init(FAKE, FAKE, FAKE, 300, 100, None) == DG_EUNSUPPORTED
    assert lib.dg_synth_logits(FAKE, FAKE, FAKE, FAKE, FAKE, 1000, 16, 100, None) == DG_EINVAL
    assert lib.dg_philox_fill(FAKE, 6, 1, 0, 0, 0, None) == DG_EINVAL
    assert lib.dg_kv_append(FAKE, FAKE, FAKE, FAKE, 0, 16, 16, 8, 64, 9, None) == DG_EUNSUPPORTED
    # the prefix buffer must hold n_prefix + n_canvas rows
    assert lib.dg_kv_append(FAKE, FAKE, FAKE, FAKE, 4096, 4096 + 255, 256, 8, 128, 1, None) == DG_EINVAL
    assert b"capacity" in lib.dg_last_error()
    assert lib.dg_kv_append(FAKE, FAKE, FAKE, FAKE, -1, 4096, 256, 8, 128, 1, None) == DG_EINVAL
    h = ctypes.c_void_p()
    assert lib.dg_step_graph_create(None, None, None, None, None, None, 0, 8, 8, 64, 1, 0.0,
                                    None, None, None, None, None, None, None, None, 16, 100, 64,
                                    None, 0, ctypes.byref(h)) == DG_EINVAL
    assert h.value is None
    assert lib.dg_status_string(-3) == b"workspace too small"


def test_ctrl_layout_matches_header():
    from block_text_diffusion_amd._lib import DgCtrl
    assert ctypes.sizeof(DgCtrl) == 40
    assert DgCtrl.tau.offset == 24 and DgCtrl.seed.offset == 0


def samp_eb(lib, **kw):
    a = dict(l=FAKE, e=FAKE, ids=FAKE, acc=FAKE, z=FAKE, ent=None, amax=FAKE, st=FAKE, ctrl=FAKE,
             budget=0.1, stop=0.005, n=16, v=1000, d=64, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.dg_sampler_step_eb(a["l"], a["e"], a["ids"], a["acc"], a["z"], a["ent"], a["amax"], a["st"],
                                  a["ctrl"], a["budget"], a["stop"], a["n"], a["v"], a["d"], a["ws"],
                                  a["wsb"], a["stream"])


def test_entropy_bounded_sampler_argument_errors(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    assert samp_eb(lib, l=None) == DG_EINVAL
    assert samp_eb(lib, amax=None) == DG_EINVAL
    assert samp_eb(lib, st=None) == DG_EINVAL
    assert samp_eb(lib, budget=-1.0) == DG_EINVAL
    assert samp_eb(lib, budget=float("nan")) == DG_EINVAL
    assert samp_eb(lib, stop=float("inf")) == DG_EINVAL
    assert samp_eb(lib, n=300) == DG_EUNSUPPORTED
    assert samp_eb(lib, wsb=16) == DG_EWORKSPACE


def test_eb_status_layout_matches_header():
    from block_text_diffusion_amd._lib import DgEbStatus
    assert ctypes.sizeof(DgEbStatus) == 16
    assert DgEbStatus.mean_entropy.offset == 8 and DgEbStatus.n_defined.offset == 12


def test_attention_ex_flags(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, 8, 4, 64, 1, 0.0]
    assert lib.dg_canvas_attention_ex(*a, 2, FAKE, 0, None) == DG_EINVAL     # unknown flag bit
    assert b"flag" in lib.dg_last_error()
    assert lib.dg_canvas_attention_ex(*a[:6], 0, 8, 8, 4, 64, 1, 0.0, 1, FAKE, 0, None) == DG_EINVAL


def test_batched_sampler_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    one = lib.dg_sampler_workspace_bytes(256, 262144, 3072)
    four = lib.dg_sampler_workspace_bytes_batched(256, 4, 262144, 3072)
    assert lib.dg_sampler_workspace_bytes_batched(256, 1, 262144, 3072) == one and four > 3 * one
    assert lib.dg_sampler_workspace_bytes_batched(256, 0, 1000, 64) == 0
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE]
    assert lib.dg_sampler_step_batched(*a, 16, 0, 1000, 64, FAKE, 0, None) == DG_EINVAL
    assert lib.dg_sampler_step_batched(*a, 256, 64, 262144, 64, FAKE, 0, None) == DG_EUNSUPPORTED  # > 2^32 bytes
    assert lib.dg_sampler_step_batched(*a, 16, 4, 1000, 64, FAKE, 16, None) == DG_EWORKSPACE
    # more than 65535 rows over the batch (small vocabulary, many canvases): refused on the host,
    # before the per-row launch grids would exceed their y extent
    assert lib.dg_sampler_workspace_bytes_batched(256, 256, 64, 64) == 0
    assert lib.dg_sampler_workspace_bytes_batched(255, 257, 64, 64) > 0
    assert lib.dg_sampler_step_batched(*a, 256, 256, 64, 64, FAKE, 1 << 40, None) == DG_EUNSUPPORTED
    assert b"rows" in lib.dg_last_error()
    assert lib.dg_sampler_workspace_bytes_topk(256, 256, 64, 64, 8) == 0


def test_topk_sampler_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    w = lib.dg_sampler_workspace_bytes_topk(256, 1, 262144, 3072, 64)
    # the top-k workspace holds candidates, lists and one partial z, far below the full sampler's
    assert 0 < w < lib.dg_sampler_workspace_bytes(256, 262144, 3072) // 10 and w % 256 == 0
    assert lib.dg_sampler_workspace_bytes_topk(256, 1, 262144, 3072, 0) == 0
    assert lib.dg_sampler_workspace_bytes_topk(256, 1, 262144, 3072, 257) == 0
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE]
    assert lib.dg_sampler_step_topk(*a, 16, 1, 1000, 64, 0, FAKE, 1 << 30, None) == DG_EINVAL
    assert lib.dg_sampler_step_topk(*a, 16, 1, 1000, 64, 257, FAKE, 1 << 30, None) == DG_EUNSUPPORTED
    # 132 sub-slices of 4096 ids times 256 candidates exceed what one row pass holds
    assert lib.dg_sampler_step_topk(*a, 1, 1, 16384 * 33, 64, 256, FAKE, 1 << 30, None) == DG_EUNSUPPORTED
    assert b"top_k" in lib.dg_last_error()
    assert lib.dg_sampler_step_topk(*a, 16, 1, 1000, 64, 8, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_sampler_step_topk(None, *a[1:], 16, 1, 1000, 64, 8, FAKE, 1 << 30, None) == DG_EINVAL
    e = [FAKE] * 9
    assert lib.dg_sampler_step_eb_topk(*e, 0.1, 0.005, 16, 1, 1000, 64, 8, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_sampler_step_eb_topk(*e, -0.1, 0.005, 16, 1, 1000, 64, 8, FAKE, 1 << 30, None) == DG_EINVAL
    assert lib.dg_sampler_step_eb_topk(*e, 0.1, 0.005, 16, 1, 1000, 64, 300, FAKE, 1 << 30, None) == DG_EUNSUPPORTED


def test_fp8_attention_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_FP8_E4M3
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, 8, 4, 64, 0.0]
    big = 1 << 30
    assert lib.dg_canvas_attention_fp8(*a, 1.0, 1.0, 1.0, 0, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_canvas_attention_fp8(*a, 0.0, 1.0, 1.0, 0, FAKE, big, None) == DG_EINVAL
    assert lib.dg_canvas_attention_fp8(*a, 1.0, float("inf"), 1.0, 0, FAKE, big, None) == DG_EINVAL
    assert lib.dg_canvas_attention_fp8(*a, 1.0, 1.0, -2.0, 0, FAKE, big, None) == DG_EINVAL
    assert lib.dg_canvas_attention_fp8(*a, 1.0, 1.0, 1.0, 4, FAKE, big, None) == DG_EINVAL    # unknown flag
    assert lib.dg_canvas_attention_fp8(*a[:10], 96, 0.0, 1.0, 1.0, 1.0, 0, FAKE, big, None) == DG_EUNSUPPORTED
    # the bf16 entry points do not take FP8 (no scales there)
    assert lib.dg_canvas_attention_ex(*a[:11], DG_FP8_E4M3, 0.0, 0, FAKE, big, None) == DG_EINVAL
    assert b"fp8" in lib.dg_last_error()


def test_entropy_bounded_step_and_graph_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_FP8_E4M3
    a = [FAKE] * 6 + [64, 8, 8, 64, 1, 0.0] + [FAKE] * 9
    assert lib.dg_denoise_step_eb(*a, 0.1, 0.005, 16, 1000, 64, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_denoise_step_eb(*a, -1.0, 0.005, 16, 1000, 64, FAKE, 1 << 30, None) == DG_EINVAL
    b = list(a)
    b[10] = DG_FP8_E4M3
    assert lib.dg_denoise_step_eb(*b, 0.1, 0.005, 16, 1000, 64, FAKE, 1 << 30, None) == DG_EUNSUPPORTED
    assert lib.dg_step_graph_create_eb(*a, 0.1, 0.005, 16, 1000, 64, FAKE, 1 << 30, None) == DG_EINVAL


def test_vocabulary_splits_beyond_the_combine_limit_are_refused(lib):
    """A vocabulary above 4194304 ids needs more than 256 vocabulary splits, more
    merge weights than the combine kernel holds: every full-sampler entry point
    refuses it on the host, and the workspace queries return 0."""
    from block_text_diffusion_amd._lib import DG_EUNSUPPORTED
    v = 8388608
    assert lib.dg_sampler_workspace_bytes(1, v, 64) == 0
    assert lib.dg_sampler_workspace_bytes_batched(1, 1, v, 64) == 0
    assert lib.dg_denoise_workspace_bytes(1, 0, 8, 8, 64, v, 64) == 0
    # the largest vocabulary that still fits is accepted by the query
    assert lib.dg_sampler_workspace_bytes(1, 4194304, 64) > 0
    big = 1 << 40
    assert samp(lib, n=1, v=v, d=64, wsb=big) == DG_EUNSUPPORTED
    assert b"splits" in lib.dg_last_error()
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE]
    assert lib.dg_sampler_step_batched(*a, 1, 1, v, 64, FAKE, big, None) == DG_EUNSUPPORTED
    assert samp_eb(lib, n=1, v=v, d=64, wsb=big) == DG_EUNSUPPORTED
    d = [FAKE] * 6 + [0, 8, 8, 64, 1, 0.0] + [FAKE] * 8
    assert lib.dg_denoise_step(*d, 1, v, 64, FAKE, big, None) == DG_EUNSUPPORTED
    e = [FAKE] * 6 + [0, 8, 8, 64, 1, 0.0] + [FAKE] * 9
    assert lib.dg_denoise_step_eb(*e, 0.1, 0.005, 1, v, 64, FAKE, big, None) == DG_EUNSUPPORTED
    h = ctypes.c_void_p()
    assert lib.dg_step_graph_create(*d, 1, v, 64, FAKE, big, ctypes.byref(h)) == DG_EUNSUPPORTED
    assert h.value is None
    assert lib.dg_step_graph_create_eb(*e, 0.1, 0.005, 1, v, 64, FAKE, big, ctypes.byref(h)) == DG_EUNSUPPORTED


def test_binding_cross_checks_attention_tensors():
    """The binding's cross-tensor checks (run before the C call, on any device):
    one dtype for Q/K/V, matching heads and head_dim, and the output's shape."""
    import torch
    import block_text_diffusion_amd as dg
    bf = torch.bfloat16
    q = torch.zeros(16, 8, 64, dtype=bf)
    kc = torch.zeros(16, 4, 64, dtype=bf)
    kp = torch.zeros(8, 4, 64, dtype=bf)
    assert dg._check_attention_tensors(q, kp, kp, kc, kc, None) == (16, 8, 4, 64, 8)
    assert dg._check_attention_tensors(q, None, None, kc, kc, None) == (16, 8, 4, 64, 0)
    with pytest.raises(ValueError, match="dtype"):
        dg._check_attention_tensors(q.float(), kp, kp, kc, kc, None)
    with pytest.raises(ValueError, match="dtype"):
        dg._check_attention_tensors(q, kp.float(), kp.float(), kc, kc, None)
    with pytest.raises(ValueError, match="canvas K/V"):
        dg._check_attention_tensors(q, kp, kp, kc, torch.zeros(16, 4, 128, dtype=bf), None)
    with pytest.raises(ValueError, match="canvas K/V"):
        dg._check_attention_tensors(q, kp, kp, torch.zeros(15, 4, 64, dtype=bf), torch.zeros(15, 4, 64, dtype=bf),
                                    None)
    with pytest.raises(ValueError, match="prefix"):
        dg._check_attention_tensors(q, kp, torch.zeros(9, 4, 64, dtype=bf), kc, kc, None)
    with pytest.raises(ValueError, match="prefix"):
        dg._check_attention_tensors(q, torch.zeros(8, 2, 64, dtype=bf), torch.zeros(8, 2, 64, dtype=bf), kc, kc,
                                    None)
    with pytest.raises(ValueError, match="out"):
        dg._check_attention_tensors(q, kp, kp, kc, kc, torch.zeros(16, 8, 32))
    with pytest.raises(ValueError, match="out"):
        dg._check_attention_tensors(q, kp, kp, kc, kc, torch.zeros(16, 8, 64, dtype=bf))
    qb, kcb, kpb = q[None].repeat(2, 1, 1, 1), kc[None].repeat(2, 1, 1, 1), kp[None].repeat(2, 1, 1, 1)
    assert dg._check_attention_tensors(qb, kpb, kpb, kcb, kcb, None, batched=True) == (16, 8, 4, 64, 8)
    with pytest.raises(ValueError, match="canvas K/V"):
        dg._check_attention_tensors(qb, kpb, kpb, kcb[:1], kcb[:1], None, batched=True)


def test_noalloc_attention_arguments(lib):
    """The no-allocation attention variant: the static scratch size, the same
    argument checks as dg_canvas_attention_ex, and sizes beyond the scratch
    refused before any HIP call."""
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_F32, DG_FP8_E4M3
    assert lib.dg_static_scratch_bytes() == 64 << 20
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert lib.dg_canvas_attention_noalloc(None, *a[1:], 16, 8, 8, 4, 64, 1, 0.0, 0, None) == DG_EINVAL
    assert lib.dg_canvas_attention_noalloc(*a, 16, 8, 8, 4, 96, 1, 0.0, 0, None) == DG_EUNSUPPORTED
    assert lib.dg_canvas_attention_noalloc(*a, 16, 8, 8, 4, 64, 1, 0.0, 2, None) == DG_EINVAL   # unknown flag
    assert lib.dg_canvas_attention_noalloc(*a, 16, 8, 8, 4, 64, DG_FP8_E4M3, 0.0, 0, None) == DG_EINVAL
    assert lib.dg_canvas_attention_noalloc(MIS, *a[1:], 16, 8, 8, 4, 64, 1, 0.0, 0, None) == DG_EINVAL
    # float32 K/V are copied to bf16 in the workspace: a 500000-row prefix needs
    # far more than the 64 MiB scratch
    need = lib.dg_attention_workspace_bytes(256, 500000, 16, 8, 128)
    assert need > 64 << 20
    assert lib.dg_canvas_attention_noalloc(*a, 256, 500000, 16, 8, 128, DG_F32, 0.0, 0, None) == DG_EUNSUPPORTED
    assert b"static scratch" in lib.dg_last_error()
    # the long-context shape fits
    assert lib.dg_attention_workspace_bytes(256, 4096, 16, 8, 128) <= 64 << 20


def test_fp8_step_and_graph_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    att = [FAKE] * 6 + [64, 8, 8, 64, 0.0]
    smp = [FAKE] * 8
    big = 1 << 30
    assert lib.dg_denoise_step_fp8(*att, 1.0, 1.0, 1.0, *smp, 16, 1000, 64, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_denoise_step_fp8(*att, 0.0, 1.0, 1.0, *smp, 16, 1000, 64, FAKE, big, None) == DG_EINVAL
    assert lib.dg_denoise_step_fp8(*att, 1.0, float("nan"), 1.0, *smp, 16, 1000, 64, FAKE, big, None) == DG_EINVAL
    bad_d = [FAKE] * 6 + [64, 8, 8, 96, 0.0]
    assert lib.dg_denoise_step_fp8(*bad_d, 1.0, 1.0, 1.0, *smp, 16, 1000, 64, FAKE, big, None) == DG_EUNSUPPORTED
    assert lib.dg_denoise_step_fp8(*att, 1.0, 1.0, 1.0, *smp, 300, 1000, 64, FAKE, big, None) == DG_EUNSUPPORTED
    h = ctypes.c_void_p()
    assert lib.dg_step_graph_create_fp8(*att, 1.0, 1.0, 1.0, None, *smp[1:], 16, 1000, 64, FAKE, big,
                                        ctypes.byref(h)) == DG_EINVAL
    assert h.value is None


def test_float32_table_sampler_arguments(lib):
    from block_text_diffusion_amd._lib import DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE]
    assert lib.dg_sampler_step_f32(*a, 16, 1000, 64, FAKE, 16, None) == DG_EWORKSPACE
    assert lib.dg_sampler_step_f32(*a, 16, 1000, 66, FAKE, 1 << 30, None) == DG_EUNSUPPORTED   # d % 4
    assert lib.dg_sampler_step_f32(*a, 1, 8388608, 64, FAKE, 1 << 40, None) == DG_EUNSUPPORTED  # splits
    assert lib.dg_sampler_step_f32(None, *a[1:], 16, 1000, 64, FAKE, 1 << 30, None) == DG_EINVAL
