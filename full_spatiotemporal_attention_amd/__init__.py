"""3D-RoPE full spatiotemporal attention on MI355X (gfx950): Python binding of libstattn.

Each function checks tensor types, marshals device pointers and the current HIP stream, and calls
the C ABI in include/st_attn.h; every arithmetic step runs in the library's HIP kernels.  PyTorch
supplies device memory and the stream only.  Tensors are [N, heads, d], contiguous, on one GPU,
with N = T*H*W video rows (t slowest, w fastest) followed by ``n_text`` text rows.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import StError  # noqa: F401

__all__ = [
    "StError",
    "attn3d",
    "attn3d_fused",
    "attn3d_stage",
    "attn3d_attend",
    "attn_factorized",
    "rope3d_apply",
    "rope3d_table",
    "attn3d_workspace_bytes",
    "attn_factorized_workspace_bytes",
    "rope3d_table_bytes",
    "library_path",
    "version",
]

WAN_SPLIT = (44, 42, 42)
HUNYUAN_SPLIT = (16, 56, 56)

_DTYPES = {torch.bfloat16: _lib.ST_BF16, torch.float32: _lib.ST_F32}


def library_path() -> str:
    _lib.load()
    return _lib.LIB_PATH


def version() -> str:
    return _lib.load().st_version().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"dtype {t.dtype} not supported (bfloat16 or float32)")
    return _DTYPES[t.dtype]


def _check_tensors(grid, n_text, *ts):
    T, H, W = (int(x) for x in grid)
    n = T * H * W + int(n_text)
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU")
        if t.device != ref.device or t.dtype != ref.dtype:
            raise ValueError("tensors must share device and dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [N, heads, d]")
        if t.dim() != 3 or t.shape != ref.shape:
            raise ValueError(f"expected equal [N, heads, d] shapes, got {tuple(t.shape)}")
    if ref.shape[0] != n:
        raise ValueError(f"grid {grid} with {n_text} text rows needs N = {n}, got {ref.shape[0]}")
    return T, H, W, ref.shape[1], ref.shape[2]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def rope3d_table_bytes(grid, rope_split=WAN_SPLIT) -> int:
    T, H, W = (int(x) for x in grid)
    return int(_lib.load().st_rope3d_table_bytes(T, H, W, _lib.split_arg(rope_split)))


def attn3d_workspace_bytes(grid, heads, n_text=0, d=128, rope_split=WAN_SPLIT,
                           dtype=torch.bfloat16) -> int:
    T, H, W = (int(x) for x in grid)
    return int(_lib.load().st_attn3d_workspace_bytes(T, H, W, int(n_text), int(heads), int(d),
                                                     _lib.split_arg(rope_split), _DTYPES[dtype]))


def attn_factorized_workspace_bytes(grid, heads, d=128, rope_split=WAN_SPLIT,
                                    dtype=torch.bfloat16) -> int:
    T, H, W = (int(x) for x in grid)
    code = _DTYPES[dtype]
    return int(_lib.load().st_attn_factorized_workspace_bytes(
        T, H, W, int(heads), int(d), _lib.split_arg(rope_split), code))


def _workspace(nbytes: int, device, workspace=None) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def rope3d_table(grid, rope_split=WAN_SPLIT, theta=10000.0, device=None) -> torch.Tensor:
    """Build the angle table for a grid and split (a uint8 device tensor)."""
    lib = _lib.load()
    T, H, W = (int(x) for x in grid)
    nbytes = rope3d_table_bytes(grid, rope_split)
    if nbytes == 0:
        raise ValueError("invalid grid or split")
    dev = torch.device("cuda") if device is None else torch.device(device)
    table = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = lib.st_rope3d_table_build(T, H, W, _lib.split_arg(rope_split), float(theta),
                                   table.data_ptr(), nbytes, _stream(dev))
    _lib.check("st_rope3d_table_build", st)
    return table


def attn3d(q, k, v, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None,
           workspace=None) -> torch.Tensor:
    """Full 3D attention: softmax(R q (R k)^T / sqrt(d)) v over all T*H*W + n_text rows."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(grid, n_text, q, out)
    nbytes = attn3d_workspace_bytes(grid, heads, n_text, d, rope_split, q.dtype)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn3d_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, int(n_text), heads,
                           d, _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                           ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                           _stream(q.device))
    _lib.check("st_attn3d_fwd", st)
    return out


def attn3d_fused(q, k, v, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                 workspace=None) -> torch.Tensor:
    """The same attention with K rotated (and V transposed) inside every tile load."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(grid, n_text, q, out)
    nbytes = int(lib.st_attn3d_fused_workspace_bytes(T, H, W, _lib.split_arg(rope_split)))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn3d_fwd_fused(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, int(n_text),
                                 heads, d, _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                                 ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                                 _stream(q.device))
    _lib.check("st_attn3d_fwd_fused", st)
    return out


def attn3d_stage(k, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0,
                 workspace=None) -> torch.Tensor:
    """First step of the bf16 path: angle table and rotated fp16 K tiles in a workspace."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, k)
    nbytes = attn3d_workspace_bytes(grid, heads, n_text, d, rope_split, k.dtype)
    ws = _workspace(nbytes, k.device, workspace)
    st = lib.st_attn3d_stage(k.data_ptr(), T, H, W, int(n_text), heads, d,
                             _lib.split_arg(rope_split), float(theta), _dtype_code(k),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(k.device))
    _lib.check("st_attn3d_stage", st)
    return ws


def attn3d_attend(q, v, grid, workspace, n_text=0, rope_split=WAN_SPLIT, out=None) -> torch.Tensor:
    """Second step of the bf16 path: attention of q against a staged workspace, values v."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, q, v)
    if out is None:
        out = torch.empty_like(q)
    st = lib.st_attn3d_attend(q.data_ptr(), v.data_ptr(), T, H, W, int(n_text), heads, d,
                              _lib.split_arg(rope_split), _dtype_code(q), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), out.data_ptr(),
                              _stream(q.device))
    _lib.check("st_attn3d_attend", st)
    return out


def attn_factorized(q, k, v, grid, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                    workspace=None) -> torch.Tensor:
    """Spatial (inside each frame) then temporal (along time at each position) attention."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, 0, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    nbytes = attn_factorized_workspace_bytes(grid, heads, d, rope_split, q.dtype)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn_factorized_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, heads, d,
                                    _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                                    ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                                    _stream(q.device))
    _lib.check("st_attn_factorized_fwd", st)
    return out


def rope3d_apply(x, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                 workspace=None) -> torch.Tensor:
    """Stand-alone 3D RoPE of every row (text rows copied); ``out=x`` rotates in place."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, x)
    if out is None:
        out = torch.empty_like(x)
    nbytes = rope3d_table_bytes(grid, rope_split)
    ws = _workspace(nbytes, x.device, workspace)
    st = lib.st_rope3d_apply(x.data_ptr(), out.data_ptr(), T, H, W, int(n_text), heads, d,
                             _lib.split_arg(rope_split), float(theta), _dtype_code(x),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(x.device))
    _lib.check("st_rope3d_apply", st)
    return out
