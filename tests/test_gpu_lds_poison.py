"""LDS-poison debug build against the normal build: every output equal bit for bit.

libstattn_ldspoison.so is the same sources built with ST_LDS_POISON: before each HBM -> LDS tile
copy, the lanes that issue it store all-ones bits (NaN as fp16, bf16 and fp32) where the copy will
land and wait for that store.  A kernel whose reads of a tile are not all ordered after the tile's
copy (a missing vmcnt wait or barrier) would read poison in that build and pass NaN to its output,
where the normal build reads the previous tile's values and may stay close to the oracle.  The
poison stores change no arithmetic, so both builds must give identical bits.

Covered, each through the C ABI: the fast launch (unsplit, key split, windows, cross-attention),
the running-max kernel (small grids, partial results, fused K rotation), the factorised path (its
spatial launch and the short temporal kernel, whose V rows arrive by the same copies) and the QKV
projection (tiles of x and w, and its table copy).  The two-block temporal kernel (T' = 33) also
depends on a barrier: each wave of a pair copies half of the value rows the other reads.  The fp32 kernel and the long temporal kernel
stage through registers within one wave (no copy to wait for) and are not affected by the flag.
"""
import os

import numpy as np
import pytest
import torch

import full_spatiotemporal_attention_amd as fa
from full_spatiotemporal_attention_amd import _lib
from st_inputs import make_qkv
from parity_util import log, to_device

pytestmark = pytest.mark.gpu

WAN = (44, 42, 42)
HUN = (16, 56, 56)


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()
    if not os.path.exists(_lib.POISON_LIB_PATH):
        raise ImportError(f"{_lib.POISON_LIB_PATH} is missing: build it with "
                          "`python -m full_spatiotemporal_attention_amd.build`")
    normal = _lib.load().st_version().decode()
    with _lib.use_library(_lib.POISON_LIB_PATH) as dbg:
        poison = dbg.st_version().decode()
    log(f"  normal build {_lib.LIB_PATH} ({normal}); poison build {_lib.POISON_LIB_PATH} ({poison})")
    if poison != normal + "+ldspoison":
        raise RuntimeError(f"the two builds come from different sources ({normal} vs {poison}): "
                           "rebuild both with `python -m full_spatiotemporal_attention_amd.build`")


def both_builds(fn):
    """fn() with the normal library, then with the poison build; both results on the host."""
    def host(r):
        r = r if isinstance(r, tuple) else (r,)
        return tuple(t.detach().cpu() for t in r)
    ref = host(fn())
    torch.cuda.synchronize()
    with _lib.use_library(_lib.POISON_LIB_PATH):
        got = host(fn())
        torch.cuda.synchronize()
    return ref, got


def assert_same(ref, got, what):
    assert len(ref) == len(got)
    for i, (a, b) in enumerate(zip(ref, got)):
        finite = bool(torch.isfinite(a.float()).all())
        assert finite, f"{what}: the normal build's output {i} is not finite (inputs are finite)"
        nan = int(torch.isnan(b.float()).sum())
        same = torch.equal(a, b)
        log(f"    {what} output {i}: shape {tuple(a.shape)}, poison NaNs {nan}, identical {same}")
        assert nan == 0, f"{what}: {nan} NaNs in the poison build's output {i}"
        assert same, f"{what}: poison build differs from the normal build in output {i}"


@pytest.mark.parametrize("grid,n_text,heads,split,what", [
    ((3, 5, 7), 9, 2, WAN, "running-max kernel alone"),
    ((8, 32, 64), 0, 2, WAN, "fast launch and guard"),
    ((5, 30, 52), 0, 12, WAN, "fast launch with key split and merge"),
    ((4, 10, 13), 37, 3, HUN, "running-max kernel, text rows, ragged tiles"),
])
def test_full_attention(grid, n_text, heads, split, what):
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  attn3d {what}: grid={grid} n_text={n_text} heads={heads} split={split} seed=9100")
    q, k, v = to_device(make_qkv(n, heads, 128, 9100, "bf16"))
    ref, got = both_builds(lambda: fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split))
    assert_same(ref, got, f"attn3d {grid}")


def test_fused_rotation():
    grid, n_text, heads = (3, 8, 12), 5, 2
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  attn3d_fused grid={grid} n_text={n_text} heads={heads} seed=9110")
    q, k, v = to_device(make_qkv(n, heads, 128, 9110, "bf16"))
    ref, got = both_builds(lambda: fa.attn3d_fused(q, k, v, grid, n_text=n_text))
    assert_same(ref, got, "attn3d_fused")


@pytest.mark.parametrize("grid,heads", [((21, 30, 52), 12), ((5, 9, 11), 2),
                                        ((33, 9, 9), 3)])   # T' = 33: two waves share V in LDS
def test_factorized(grid, heads):
    n = grid[0] * grid[1] * grid[2]
    log(f"  attn_factorized grid={grid} heads={heads} seed=9120")
    q, k, v = to_device(make_qkv(n, heads, 128, 9120, "bf16"))
    ref, got = both_builds(lambda: fa.attn_factorized(q, k, v, grid))
    assert_same(ref, got, f"attn_factorized {grid}")


@pytest.mark.parametrize("grid,window,heads", [
    ((4, 6, 8), (2, 3, 4), 2),          # running-max kernel
    ((14, 30, 52), (7, 15, 26), 2),     # fast launch, ragged key tile
])
def test_windows(grid, window, heads):
    n = grid[0] * grid[1] * grid[2]
    log(f"  attn_window grid={grid} window={window} heads={heads} seed=9130")
    q, k, v = to_device(make_qkv(n, heads, 128, 9130, "bf16"))
    ref, got = both_builds(lambda: fa.attn_window(q, k, v, grid, window))
    assert_same(ref, got, f"attn_window {window}")


@pytest.mark.parametrize("n_q,n_kv,heads", [(1000, 77, 2), (32760, 512, 12)])
def test_cross_attention(n_q, n_kv, heads):
    log(f"  attn_cross n_q={n_q} n_kv={n_kv} heads={heads} seed=9140")
    q = to_device(make_qkv(n_q, heads, 128, 9140, "bf16"))[0]
    _, k, v = to_device(make_qkv(n_kv, heads, 128, 9141, "bf16"))
    ref, got = both_builds(lambda: fa.attn_cross(q, k, v))
    assert_same(ref, got, "attn_cross")


def test_partial_results():
    grid, heads = (3, 6, 9), 2
    n = grid[0] * grid[1] * grid[2]
    log(f"  attn3d_partial grid={grid} heads={heads} rows [40, 140) x keys [17, 150) seed=9150")
    q, k, v = to_device(make_qkv(n, heads, 128, 9150, "bf16"))
    ref, got = both_builds(lambda: fa.attn3d_partial(q[40:140], k[17:150], v[17:150], grid,
                                                     q_begin=40, kv_begin=17))
    assert_same(ref, got, "attn3d_partial")


@pytest.mark.parametrize("grid,n_text,heads", [((3, 5, 7), 9, 2), ((21, 30, 52), 0, 12)])
def test_qkv_projection(grid, n_text, heads):
    n = grid[0] * grid[1] * grid[2] + n_text
    c = heads * 128
    log(f"  qkv_rope grid={grid} n_text={n_text} heads={heads} seed=9160")
    g = torch.Generator().manual_seed(9160)
    x = torch.randn(n, c, generator=g).to(torch.bfloat16).cuda()
    w = (torch.randn(3 * c, c, generator=g) / np.sqrt(c)).to(torch.bfloat16).cuda()
    b = (0.1 * torch.randn(3 * c, generator=g)).to(torch.bfloat16).cuda()
    ref, got = both_builds(lambda: fa.qkv_rope(x, w, grid, bias=b, n_text=n_text))
    assert_same(ref, got, "qkv_rope")
