"""Build libdg.so (the HIP kernels plus the C ABI) in-tree for gfx950.

    python -m block_text_diffusion_amd.build [--isa]

--isa also keeps the gfx950 assembly of every kernel file under _build/ so
register counts, spills and LDS use can be read.
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdg.so")

SOURCES = ["attention.hip", "sampler.hip", "decode.hip", "dg_api.cpp"]

HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libdg.so")
    return path


def _compile(src, isa):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPFLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[cmd.index("-c"):cmd.index("-c")] = ["-x", "hip"]
    if isa and src.endswith(".hip"):
        cmd += ["-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(isa=False, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, isa), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libdg_asan.so")


def asan_runtime():
    """The clang AddressSanitizer runtime that a host process must preload to load ASAN_LIB."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(llvm, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[-1]


def build_asan(verbose=False):
    """A variant of libdg.so whose host code (the C ABI: argument validation,
    workspace planning, launch sequencing) is built with AddressSanitizer, for
    running the CPU ABI tests under it.  Device code is built as usual.  Not
    the product library; it lives under _build/asan."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPFLAGS, *asan, "-g", "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[cmd.index("-c"):cmd.index("-c")] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True, cwd=ASAN_DIR)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed for {src}:\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", *objs, "-o", ASAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{res.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", action="store_true")
    ap.add_argument("--asan", action="store_true", help="also build the AddressSanitizer variant (_build/asan)")
    a = ap.parse_args()
    build(isa=a.isa, verbose=True)
    if a.asan:
        build_asan(verbose=True)
    sys.exit(0)
