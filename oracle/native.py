"""ctypes access to oracle/philox_c.c (test infrastructure only).

The C file is compiled with gcc into oracle/_philox_c.so on first use (or by
__graft_entry__.build()).  Functions return None when no C compiler is
available, and the numpy paths in oracle.philox / oracle.synth are used instead.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_c.c")
LIB = os.path.join(HERE, "_philox_c.so")
_lib = None


def build(force=False):
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        return None
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"],
                   check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        path = build()
        if path is None:
            return None
        L = ctypes.CDLL(path)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
        L.dg_oracle_philox.argtypes = [u32p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32, u32p]
        L.dg_oracle_gumbel_scores.argtypes = [f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_uint64, ctypes.c_uint32, i64p, f32p]
        L.dg_oracle_synth_noise.argtypes = [f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                            ctypes.c_uint32, i64p, f32p]
        _lib = L
    return _lib


def philox(ctr, k0, k1):
    L = lib()
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    out = np.empty_like(ctr)
    L.dg_oracle_philox(ctr, len(ctr), k0, k1, out)
    return out


def gumbel_scores(logits, inv_t, seed, gstep, positions):
    L = lib()
    if L is None:
        return None
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    out = np.empty_like(logits)
    L.dg_oracle_gumbel_scores(logits, logits.shape[0], logits.shape[1], float(inv_t),
                              int(seed) & 0xFFFFFFFFFFFFFFFF, int(gstep), pos, out)
    return out


def synth_noise(table, n_rows, vocab, seed, gstep, positions):
    L = lib()
    if L is None:
        return None
    table = np.ascontiguousarray(table, dtype=np.float32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    out = np.empty((len(pos), vocab), dtype=np.float32)
    L.dg_oracle_synth_noise(table, len(pos), vocab, int(seed) & 0xFFFFFFFFFFFFFFFF, int(gstep), pos, out)
    return out
