"""ctypes view of libdg.so (the C ABI declared in include/dg.h).

Argument marshalling only: every step of the denoising path runs in the HIP
kernels behind these symbols.  The library must be built first
(``python -m block_text_diffusion_amd.build``); loading fails loudly if it is
missing, and there is no fallback implementation.
"""
import ctypes
import os

# DG_LIBRARY may name another build of the same sources (the AddressSanitizer
# variant the CPU ABI tests run under); by default the in-tree libdg.so.
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")

DG_OK = 0
DG_EINVAL = -1
DG_EUNSUPPORTED = -2
DG_EWORKSPACE = -3
DG_EHIP = -4
DG_F32 = 0
DG_BF16 = 1
DG_FP8_E4M3 = 2
DG_GUMBEL = 1
DG_COMMIT_ONLY = 2
DG_AUTO_ADVANCE = 4
DG_T_SCHEDULE = 8
DG_ATTN_CAUSAL = 1


class DgCtrl(ctypes.Structure):
    """Mirror of dg_ctrl (40 bytes)."""
    _fields_ = [
        ("seed", ctypes.c_uint64),
        ("gstep", ctypes.c_uint32),
        ("s_in_block", ctypes.c_uint32),
        ("s_max", ctypes.c_uint32),
        ("flags", ctypes.c_uint32),
        ("tau", ctypes.c_float),
        ("t_start", ctypes.c_float),
        ("t_end", ctypes.c_float),
        ("reserved", ctypes.c_uint32),
    ]


assert ctypes.sizeof(DgCtrl) == 40


class DgEbStatus(ctypes.Structure):
    """Mirror of dg_eb_status (16 bytes)."""
    _fields_ = [
        ("n_accepted", ctypes.c_uint32),
        ("stop", ctypes.c_uint32),
        ("mean_entropy", ctypes.c_float),
        ("n_defined", ctypes.c_uint32),
    ]


assert ctypes.sizeof(DgEbStatus) == 16

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float
_u32 = ctypes.c_uint32

# name -> (restype, argtypes)
SIGNATURES = {
    "dg_attention_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dg_canvas_attention": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "dg_canvas_attention_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                    ctypes.c_uint32, _vp, _sz, _vp]),
    "dg_static_scratch_bytes": (_sz, []),
    "dg_canvas_attention_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                         ctypes.c_uint32, _vp]),
    "dg_attention_batched_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "dg_canvas_attention_batched": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                         _f, _vp, _sz, _vp]),
    "dg_canvas_attention_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _f, _u32,
                                     _vp, _sz, _vp]),
    "dg_sampler_workspace_bytes": (_sz, [_i, _i, _i]),
    "dg_embedding_packed_bytes": (_sz, [_i, _i]),
    "dg_embedding_pack": (_i, [_vp, _vp, _i, _i, _vp]),
    "dg_sampler_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "dg_sampler_step_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "dg_sampler_step_eb": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _i, _i, _i,
                                _vp, _sz, _vp]),
    "dg_sampler_workspace_bytes_batched": (_sz, [_i, _i, _i, _i]),
    "dg_sampler_step_batched": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "dg_sampler_step_eb_batched": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _i, _i, _i, _i,
                                        _vp, _sz, _vp]),
    "dg_sampler_workspace_bytes_topk": (_sz, [_i, _i, _i, _i, _i]),
    "dg_sampler_step_topk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "dg_sampler_step_eb_topk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _i, _i, _i, _i, _i,
                                     _vp, _sz, _vp]),
    "dg_denoise_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "dg_denoise_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "dg_denoise_step_eb": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _f, _f, _i, _i, _i, _vp, _sz, _vp]),
    "dg_denoise_step_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _f, _f, _f,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "dg_step_graph_create_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _f, _f, _f,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz,
                                      ctypes.POINTER(_vp)]),
    "dg_step_graph_create_eb": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _f, _f, _i, _i, _i, _vp, _sz, ctypes.POINTER(_vp)]),
    "dg_step_graph_create": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz,
                                  ctypes.POINTER(_vp)]),
    "dg_step_graph_launch": (_i, [_vp, _vp]),
    "dg_step_graph_destroy": (None, [_vp]),
    "dg_canvas_init": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "dg_kv_append": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "dg_synth_logits": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "dg_philox_fill": (_i, [_vp, _sz, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                            ctypes.c_uint32, _vp]),
    "dg_probe_mfma_bf16": (_i, [_vp, _i, _i, _vp]),
    "dg_probe_copy": (_i, [_vp, _vp, _sz, _vp]),
    "dg_probe_read": (_i, [_vp, _sz, _vp, _vp]),
    "dg_profile_enable": (_i, [_i]),
    "dg_profile_read": (_i, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                             ctypes.POINTER(ctypes.c_int), _i]),
    "dg_status_string": (ctypes.c_char_p, [_i]),
    "dg_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libdg.so once and attach the signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_text_diffusion_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DgError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"dg status {status} ({load().dg_status_string(status).decode()}): {detail}")


def check(status):
    if status != DG_OK:
        raise DgError(status, load().dg_last_error().decode())
    return status
