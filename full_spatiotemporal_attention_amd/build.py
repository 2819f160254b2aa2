"""Build libstattn.so in-tree with hipcc for gfx950.

Usage: ``python -m full_spatiotemporal_attention_amd.build`` (or ``build()`` from Python).  Each
HIP source is compiled to an object under ``_build/`` next to this file, then linked into
``libstattn.so`` in the package directory, which the ctypes binding loads.

``build()`` also makes (and ``build_lds_poison()`` makes alone) a debug build of the same sources,
``libstattn_ldspoison.so``, with
``ST_LDS_POISON`` defined: before every HBM -> LDS tile copy the destination bytes are first set to
all-ones (NaN in fp16, bf16 and fp32), so that a read of a tile not ordered after its copy (a
missing wait or barrier) yields NaN in the output instead of the previous tile's values.  Its
outputs must equal the normal build's bit for bit.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libstattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
POISON_LIB_PATH = os.path.join(PKG_DIR, "libstattn_ldspoison.so")
ARCH = "gfx950"

SOURCES = ["st_api.hip", "rope.hip", "attn_bf16.hip", "attn_temporal.hip", "attn_f32.hip", "merge.hip",
           "qkv_rope.hip"]

# Extra flags per source.  The flash kernels take row maxima of MFMA results with fmaxf; without
# -fno-honor-nans every operand is first canonicalised (an extra v_max_f32 x, x each).  A NaN
# input still reaches the output: it enters the exponentials and the products.
SOURCE_FLAGS = {
    "attn_bf16.hip": ["-fno-honor-nans"],
    "attn_temporal.hip": ["-fno-honor-nans"],
}

# Packed fp32 instructions are switched off for all device code (the compiler would otherwise
# form v_pk_{add,mul,fma}_f32 from scalar float code).
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_hash() -> str:
    """Hash of every source and header the library is built from (12 hex digits)."""
    h = hashlib.sha256()
    for path in ([os.path.join(CSRC, f) for f in SOURCES] + [os.path.join(CSRC, "st_internal.h"),
                                                            os.path.join(INCLUDE, "st_attn.h")]):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:12]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _build_lib(lib_path: str, obj_dir: str, extra: list, verbose: bool) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, f'-DST_SOURCE_HASH="{source_hash()}"',
               "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = lib_path + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False, lds_poison: bool = True) -> str:
    """Compile every HIP source and link libstattn.so, and (by default) the LDS-poison debug build
    beside it from the same sources; return the library path."""
    path = _build_lib(LIB_PATH, BUILD_DIR, [], verbose)
    if lds_poison:
        build_lds_poison(verbose)
    return path


def build_lds_poison(verbose: bool = False) -> str:
    """Compile the LDS-poison debug build, libstattn_ldspoison.so; return its path."""
    return _build_lib(POISON_LIB_PATH, os.path.join(BUILD_DIR, "lds_poison"), ["-DST_LDS_POISON=1"],
                      verbose)


if __name__ == "__main__":
    if "--lds-poison" in sys.argv:
        print(build_lds_poison(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
        print(POISON_LIB_PATH)
