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
    "attn3d_noalloc",
    "attn3d_stage",
    "attn3d_attend",
    "attn_factorized",
    "attn_window",
    "attn_cross",
    "attn3d_partial",
    "attn_merge",
    "qkv_rope",
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
    """Path of the loaded library: the in-tree libstattn.so, or the build STATTN_LIB names."""
    return _lib.loaded_path()


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


def _check_out(out, like, what="out"):
    """A caller-supplied output must match `like` exactly: the C ABI only sees a pointer."""
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if out.device != like.device or out.dtype != like.dtype:
        raise ValueError(f"{what} must be on {like.device} with dtype {like.dtype}")
    if out.shape != like.shape:
        raise ValueError(f"{what} must have shape {tuple(like.shape)}, got {tuple(out.shape)}")
    if not out.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return out


def _check_rows_tensors(*ts):
    """[rows, heads, d] GPU tensors sharing a device and dtype (cross and partial attention)."""
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 3:
            raise ValueError("expected contiguous [rows, heads, d] GPU tensors")
        if t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("tensors must share device and dtype")


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
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch tensor")
        if workspace.device != torch.device(device) or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
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
        _check_out(out, q)
    nbytes = attn3d_workspace_bytes(grid, heads, n_text, d, rope_split, q.dtype)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn3d_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, int(n_text), heads,
                           d, _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                           ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                           _stream(q.device))
    _lib.check("st_attn3d_fwd", st)
    return out


def attn3d_noalloc(q, k, v, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None) -> torch.Tensor:
    """attn3d without a workspace: the library's static per-device scratch (see the C header for
    its size limit and the race between overlapping calls on one GPU).  With ``out`` given, the
    call allocates nothing."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    with torch.cuda.device(q.device):   # the library's scratch is that of the tensors' device
        st = lib.st_attn3d_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, int(n_text),
                                       heads, d, _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                                       out.data_ptr(), _stream(q.device))
    _lib.check("st_attn3d_fwd_noalloc", st)
    return out


def attn3d_fused(q, k, v, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                 workspace=None) -> torch.Tensor:
    """The same attention with K rotated (and V transposed) inside every tile load."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
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
    else:
        _check_out(out, q)
    if workspace is None:
        raise ValueError("attn3d_attend needs the workspace attn3d_stage filled")
    nbytes = attn3d_workspace_bytes(grid, heads, n_text, d, rope_split, q.dtype)
    workspace = _workspace(nbytes, q.device, workspace)
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
    else:
        _check_out(out, q)
    nbytes = attn_factorized_workspace_bytes(grid, heads, d, rope_split, q.dtype)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn_factorized_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, heads, d,
                                    _lib.split_arg(rope_split), float(theta), _dtype_code(q),
                                    ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                                    _stream(q.device))
    _lib.check("st_attn_factorized_fwd", st)
    return out


def attn_window(q, k, v, grid, window, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                workspace=None) -> torch.Tensor:
    """Attention inside non-overlapping (wt, wh, ww) windows of the grid, with 3D RoPE."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, 0, q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    win = _lib.split_arg(window)
    nbytes = int(lib.st_attn3d_window_workspace_bytes(T, H, W, heads, d, _lib.split_arg(rope_split), win,
                                                      _dtype_code(q)))
    if nbytes == 0:
        raise ValueError("invalid grid, window, split or dtype for window attention")
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn3d_window_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, heads, d,
                                  _lib.split_arg(rope_split), float(theta), win, _dtype_code(q),
                                  ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                                  _stream(q.device))
    _lib.check("st_attn3d_window_fwd", st)
    return out


def rope3d_apply(x, grid, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, out=None,
                 workspace=None) -> torch.Tensor:
    """Stand-alone 3D RoPE of every row (text rows copied); ``out=x`` rotates in place."""
    lib = _lib.load()
    T, H, W, heads, d = _check_tensors(grid, n_text, x)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_out(out, x)
    nbytes = rope3d_table_bytes(grid, rope_split)
    ws = _workspace(nbytes, x.device, workspace)
    st = lib.st_rope3d_apply(x.data_ptr(), out.data_ptr(), T, H, W, int(n_text), heads, d,
                             _lib.split_arg(rope_split), float(theta), _dtype_code(x),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(x.device))
    _lib.check("st_rope3d_apply", st)
    return out


def attn_cross(q, k, v, out=None, workspace=None) -> torch.Tensor:
    """Text cross-attention: softmax(q k^T / sqrt(d)) v, q [Nq, heads, d], k/v [Nkv, heads, d]."""
    lib = _lib.load()
    _check_rows_tensors(q, k, v)
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [Nkv, heads, d] with the heads and d of q")
    n_q, heads, d = q.shape
    n_kv = k.shape[0]
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    nbytes = int(lib.st_attn_cross_workspace_bytes(n_q, n_kv, heads, d, code))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn_cross_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), n_q, n_kv, heads, d, code,
                               ws.data_ptr(), ws.numel() * ws.element_size(), out.data_ptr(),
                               _stream(q.device))
    _lib.check("st_attn_cross_fwd", st)
    return out


def attn3d_partial(q, k, v, grid, q_begin=0, kv_begin=0, n_text=0, rope_split=WAN_SPLIT,
                   theta=10000.0, workspace=None):
    """Attention of global query rows [q_begin, +len(q)) against key rows [kv_begin, +len(k)).

    Returns (out, lse): the softmax-normalised output over this run of keys and the float32
    log-sum-exp of the scaled scores, [len(q), heads].
    """
    lib = _lib.load()
    T, H, W = (int(x) for x in grid)
    _check_rows_tensors(q, k, v)
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [Nkv, heads, d] with the heads and d of q")
    q_count, heads, d = q.shape
    kv_count = k.shape[0]
    code = _dtype_code(q)
    sp = _lib.split_arg(rope_split)
    out = torch.empty_like(q)
    lse = torch.empty((q_count, heads), dtype=torch.float32, device=q.device)
    nbytes = int(lib.st_attn3d_partial_workspace_bytes(T, H, W, int(n_text), heads, d, sp, code, kv_count))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.st_attn3d_partial_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, int(n_text), heads,
                                   d, sp, float(theta), code, int(q_begin), q_count, int(kv_begin),
                                   kv_count, ws.data_ptr(), ws.numel() * ws.element_size(),
                                   out.data_ptr(), lse.data_ptr(), _stream(q.device))
    _lib.check("st_attn3d_partial_fwd", st)
    return out, lse


def attn_merge(parts, out=None, lse_out=None):
    """Merge [(o_i, lse_i), ...] over disjoint key runs; returns (out, lse)."""
    import ctypes
    lib = _lib.load()
    if not parts:
        raise ValueError("no parts")
    o0, l0 = parts[0]
    if not isinstance(o0, torch.Tensor) or o0.dim() != 3 or o0.device.type != "cuda":
        raise ValueError("parts must be [rows, heads, d] GPU tensors")
    n_rows, heads, d = o0.shape
    for o, l in parts:
        if not isinstance(o, torch.Tensor) or not isinstance(l, torch.Tensor):
            raise TypeError("parts must be (out, lse) pairs of torch tensors")
        if o.shape != o0.shape or o.dtype != o0.dtype or o.device != o0.device or not o.is_contiguous():
            raise ValueError("parts must share shape, dtype and device, and be contiguous")
        if (l.shape != (n_rows, heads) or l.dtype != torch.float32 or l.device != o0.device
                or not l.is_contiguous()):
            raise ValueError("lse parts must be contiguous float32 [rows, heads] on the parts' device")
    if out is None:
        out = torch.empty_like(o0)
    else:
        _check_out(out, o0)
    if lse_out is None:
        lse_out = torch.empty_like(l0)
    else:
        _check_out(lse_out, l0, "lse_out")
    n = len(parts)
    optr = (ctypes.c_void_p * n)(*[o.data_ptr() for o, _ in parts])
    lptr = (ctypes.c_void_p * n)(*[l.data_ptr() for _, l in parts])
    st = lib.st_attn_merge(n, optr, lptr, n_rows, heads, d, _dtype_code(o0), out.data_ptr(),
                           lse_out.data_ptr(), _stream(o0.device))
    _lib.check("st_attn_merge", st)
    return out, lse_out


def qkv_rope(x, w, grid, bias=None, n_text=0, rope_split=WAN_SPLIT, theta=10000.0, workspace=None):
    """QKV projection x w^T (+ bias) with q and k rotated by 3D RoPE; returns (q, k, v) [N, heads, d].

    x [N, C], w [3C, C] (a linear layer's weight), bias [3C] or None; C = heads * d with d the
    sum of rope_split.
    """
    lib = _lib.load()
    T, H, W = (int(a) for a in grid)
    d = int(sum(rope_split))
    for t in (x, w) + ((bias,) if bias is not None else ()):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("expected contiguous GPU tensors")
        if t.dtype != x.dtype or t.device != x.device:
            raise ValueError("x, w and bias must share a dtype and device")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    n, c = x.shape
    if w.shape != (3 * c, c) or c % d:
        raise ValueError("w must be [3C, C] and C a multiple of the head dim")
    if bias is not None and bias.shape != (3 * c,):
        raise ValueError("bias must be [3C]")
    heads = c // d
    code = _dtype_code(x)
    q = torch.empty((n, heads, d), dtype=x.dtype, device=x.device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    sp = _lib.split_arg(rope_split)
    nbytes = int(lib.st_qkv_rope_workspace_bytes(T, H, W, sp))
    ws = _workspace(nbytes, x.device, workspace)
    st = lib.st_qkv_rope_fwd(x.data_ptr(), w.data_ptr(), None if bias is None else bias.data_ptr(),
                             T, H, W, int(n_text), heads, d, sp, float(theta), code, ws.data_ptr(),
                             ws.numel() * ws.element_size(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             _stream(x.device))
    _lib.check("st_qkv_rope_fwd", st)
    return q, k, v
