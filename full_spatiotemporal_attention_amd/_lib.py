"""ctypes loader for libstattn.so (the in-tree HIP library) and its C signatures."""
from __future__ import annotations

import contextlib
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libstattn.so")
POISON_LIB_PATH = os.path.join(PKG_DIR, "libstattn_ldspoison.so")   # LDS-poison debug build

ST_OK = 0
ST_BF16 = 0
ST_F32 = 1

_STATUS_NAMES = {
    0: "ST_OK", 1: "ST_ERR_NULL", 2: "ST_ERR_SHAPE", 3: "ST_ERR_SPLIT", 4: "ST_ERR_UNSUPPORTED",
    5: "ST_ERR_WORKSPACE", 6: "ST_ERR_HIP", 7: "ST_ERR_ALIAS", 8: "ST_ERR_ALIGN",
}

_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_p = ctypes.c_void_p
_split = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes); one entry per declaration in include/st_attn.h
SIGNATURES = {
    "st_rope3d_table_bytes": (_sz, [_i, _i, _i, _split]),
    "st_rope3d_table_build": (_i, [_i, _i, _i, _split, _f, _p, _sz, _p]),
    "st_attn3d_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _split, _i]),
    "st_attn3d_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p, _p]),
    "st_attn3d_stage": (_i, [_p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p]),
    "st_attn3d_attend": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _split, _i, _p, _sz, _p, _p]),
    "st_attn3d_noalloc_scratch_bytes": (_sz, []),
    "st_attn3d_fwd_noalloc": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _p]),
    "st_attn3d_fused_workspace_bytes": (_sz, [_i, _i, _i, _split]),
    "st_attn3d_fwd_fused": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p, _p]),
    "st_attn_factorized_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _split, _i]),
    "st_attn_factorized_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p, _p]),
    "st_attn3d_window_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _split, _split, _i]),
    "st_attn3d_window_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _split, _f, _split, _i, _p, _sz, _p, _p]),
    "st_rope3d_apply": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p]),
    "st_attn_cross_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "st_attn_cross_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _sz, _p, _p]),
    "st_attn3d_partial_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _split, _i, _i]),
    "st_attn3d_partial_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _i, _i, _i, _i,
                                   _p, _sz, _p, _p, _p]),
    "st_attn_merge": (_i, [_i, ctypes.POINTER(_p), ctypes.POINTER(_p), _i, _i, _i, _i, _p, _p, _p]),
    "st_qkv_rope_workspace_bytes": (_sz, [_i, _i, _i, _split]),
    "st_qkv_rope_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _split, _f, _i, _p, _sz, _p, _p, _p, _p]),
    "st_status_str": (ctypes.c_char_p, [_i]),
    "st_last_hip_error": (_i, []),
    "st_version": (ctypes.c_char_p, []),
}


class StError(RuntimeError):
    """A libstattn call returned a status other than ST_OK."""

    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        name = _STATUS_NAMES.get(status, str(status))
        extra = f" (hipError {hip_error})" if status == 6 else ""
        super().__init__(f"{fn} failed: {name}{extra}")


_LIB = None
_LIB_LOADED_PATH = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libstattn.so once; raise if it has not been built (there is no fallback path).

    ``STATTN_LIB`` in the environment names another build of the same library (the sanitized
    debug build of build_sanitized.py); by default the in-tree libstattn.so is loaded."""
    global _LIB, _LIB_LOADED_PATH
    if _LIB is not None:
        return _LIB
    if path is None:
        path = os.environ.get("STATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m full_spatiotemporal_attention_amd.build` "
            "(hipcc, gfx950). There is no CPU or PyTorch fallback.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    _LIB_LOADED_PATH = os.path.abspath(path)
    return lib


def loaded_path() -> str:
    """Path of the library the binding calls (loading it first if needed)."""
    load()
    return _LIB_LOADED_PATH


@contextlib.contextmanager
def use_library(path: str):
    """Route every call of the binding to another build of the library inside the block (e.g.
    the LDS-poison debug build, POISON_LIB_PATH); the previous library is restored on exit."""
    global _LIB, _LIB_LOADED_PATH
    saved, saved_path = _LIB, _LIB_LOADED_PATH
    _LIB = None
    try:
        yield load(path)
    finally:
        _LIB, _LIB_LOADED_PATH = saved, saved_path


def split_arg(split) -> ctypes.Array:
    arr = (ctypes.c_int * 3)(*[int(x) for x in split])
    return arr


def check(fn: str, status: int) -> None:
    if status != ST_OK:
        raise StError(fn, status, load().st_last_hip_error() if status == 6 else 0)
