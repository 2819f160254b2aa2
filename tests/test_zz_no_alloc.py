"""The allocation-free entry point against st_attn3d_fwd, through the C ABI.

st_attn3d_fwd_noalloc runs st_attn3d_fwd's launches on the library's static per-device scratch
instead of a caller workspace, so its output must equal st_attn3d_fwd's bit for bit; two calls in a
row, the second on a smaller input, check that nothing left in the scratch by the first call leaks
into the second.  The larger case is also held to the oracle on sampled rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import full_spatiotemporal_attention_amd as fa
from full_spatiotemporal_attention_amd import _lib
from st_inputs import make_qkv, sample_rows
from parity_util import assert_close, host_f64, log, to_device

pytestmark = pytest.mark.gpu

WAN = (44, 42, 42)


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()


def _noalloc(lib, q, k, v, grid, n_text, out, dtype_code):
    T, H, W = grid
    st = lib.st_attn3d_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, W, n_text,
                                   q.shape[1], q.shape[2], _lib.split_arg(WAN), 10000.0, dtype_code,
                                   out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _lib.check("st_attn3d_fwd_noalloc", st)


def test_noalloc_matches_workspace_entry_point_twice():
    lib = _lib.load()
    # first the fast-launch case (16,384 tokens x 2 heads, several 256-row blocks, guard launch),
    # then a smaller ragged grid with text rows that runs the running-max kernel alone
    for grid, n_text, heads, seed in (((8, 32, 64), 0, 2, 801), ((5, 9, 11), 7, 3, 802)):
        n = grid[0] * grid[1] * grid[2] + n_text
        log(f"  no-alloc entry point grid={grid} n_text={n_text} heads={heads} seed={seed}")
        x = make_qkv(n, heads, 128, seed, "bf16")
        q, k, v = to_device(x)
        ref = fa.attn3d(q, k, v, grid, n_text=n_text)
        out = torch.full_like(q, float("nan"))
        _noalloc(lib, q, k, v, grid, n_text, out, _lib.ST_BF16)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        rows = sample_rows(n, grid[0] * grid[1] * grid[2], grid[1] * grid[2], 256, seed + 3)
        want = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, WAN, 10000.0, rows=rows)
        assert_close(host_f64(out)[rows], want, "bf16", f"no-alloc {grid}+{n_text}")


def test_noalloc_f32_and_binding():
    grid, heads = (3, 4, 6), 2
    x = make_qkv(72, heads, 128, 803, "f32")
    q, k, v = to_device(x)
    ref = fa.attn3d(q, k, v, grid)
    out = torch.empty_like(q)
    fa.attn3d_noalloc(q, k, v, grid, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_refuses_requests_past_its_scratch():
    lib = _lib.load()
    cap = lib.st_attn3d_noalloc_scratch_bytes()
    # 21 x 45 x 80 tokens x 12 heads needs 232 MB of staged key tiles
    grid, heads = (21, 45, 80), 12
    need = fa.attn3d_workspace_bytes(grid, heads)
    assert need > cap
    q = torch.zeros(75600, heads, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    T, H, W = grid
    st = lib.st_attn3d_fwd_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), T, H, W, 0, heads, 128,
                                   _lib.split_arg(WAN), 10000.0, _lib.ST_BF16, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 5   # ST_ERR_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
