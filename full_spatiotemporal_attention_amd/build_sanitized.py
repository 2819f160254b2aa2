"""Debug build of libstattn with AddressSanitizer and UndefinedBehaviorSanitizer on the host code.

Only the host side of each source is instrumented (every sanitizer flag goes through -Xarch_host);
the gfx950 device code is built exactly as in build.py.  The result, ``_build/sanitized/
libstattn_san.so``, is meant for the CPU-side C-ABI tests: load it in a process that has the ASan
runtime preloaded (``sanitizer_env()``) and point the binding at it with ``STATTN_LIB``.

Usage: ``python -m full_spatiotemporal_attention_amd.build_sanitized``.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as _b

OUT_DIR = os.path.join(_b.BUILD_DIR, "sanitized")
LIB_PATH = os.path.join(OUT_DIR, "libstattn_san.so")

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan", "-g"]


def asan_runtime() -> str:
    r = subprocess.run([_b.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    if not path or not os.path.exists(path):
        raise RuntimeError("ASan runtime (libclang_rt.asan-x86_64.so) not found next to hipcc")
    return path


def sanitizer_env(base=None) -> dict:
    """Environment for a child process that loads the sanitized library."""
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["STATTN_LIB"] = LIB_PATH
    return env


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = _b.hipcc()
    objs, procs = [], []
    for src in _b.SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *_b.HIPCC_FLAGS, *_b.SOURCE_FLAGS.get(src, []), *HOST_SAN,
               f'-DST_SOURCE_HASH="{_b.source_hash()}"', "-I", _b.INCLUDE,
               "-I", _b.CSRC, "-c", os.path.join(_b.CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out.decode(errors="replace")))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s} ---\n{t}" for s, t in failed))
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={_b.ARCH}", *HOST_SAN, "-o", LIB_PATH, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
