"""GPU parity: every HIP entry point against the float64 oracle on the same seeded inputs.

Small grids are compared on every output element (several 64-key tiles, 256-row query tiles and a
ragged tail); the configurations shaped like the pages' workloads are compared on a seeded sample
of query rows per head (all keys always used), in the launch configuration the bench times.
All calls go through the C ABI (ctypes) of libstattn.so.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import full_spatiotemporal_attention_amd as fa
from st_inputs import make_qkv, sample_rows
from parity_util import assert_close, errors, host_f64, log, to_device

pytestmark = pytest.mark.gpu

WAN = (44, 42, 42)
HUN = (16, 56, 56)


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()  # raises if the HIP library is missing: no fallback
    log(f"device: {torch.cuda.get_device_name(0)}  lib: {fa.library_path()}")


def run_full(grid, heads, dtype, seed, n_text=0, split=WAN, rows=None, head_subset=None,
             **gen):
    T, H, W = grid
    n = T * H * W + n_text
    log(f"  full attention grid={grid} n_text={n_text} heads={heads} dtype={dtype} split={split} "
        f"seed={seed} rows={'all' if rows is None else len(rows)}")
    x = make_qkv(n, heads, 128, seed, dtype, **gen)
    q, k, v = to_device(x)
    out = fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    got = host_f64(out)
    hsel = list(range(heads)) if head_subset is None else list(head_subset)
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0, rows=rows,
                                    heads=hsel)
    got = got[:, hsel] if rows is None else got[rows][:, hsel]
    return got, ref


# ------------------------------------------------------------------------------------------
# Angle table and stand-alone RoPE
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("grid,split", [((3, 4, 6), WAN), ((21, 30, 52), WAN),
                                        ((33, 45, 80), HUN), ((1, 1, 1), (0, 0, 128))])
def test_rope_table(grid, split):
    log(f"  table grid={grid} split={split}")
    tab = fa.rope3d_table(grid, split)
    torch.cuda.synchronize()
    got = tab.cpu().numpy().view(np.float32).reshape(-1, 2)
    freqs = oracle.rope_frequencies(split)
    want = []
    for axis, ext in enumerate(grid):
        for pos in range(ext):
            for j in range(split[axis] // 2):
                phi = pos * freqs[axis][j]
                want.append((math.cos(phi), math.sin(phi)))
    want.append((1.0, 0.0))
    want = np.array(want)
    assert np.abs(got[:len(want)] - want).max() <= 6e-8


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid,n_text,heads,split", [((3, 4, 6), 0, 2, WAN), ((5, 7, 11), 9, 3, HUN),
                                                     ((21, 30, 52), 0, 12, WAN),
                                                     ((2, 3, 4), 5, 24, HUN),    # heads in two passes of 16
                                                     ((1, 2, 3), 0, 40, WAN)])   # and three
def test_rope_apply(dtype, grid, n_text, heads, split):
    T, H, W = grid
    n = T * H * W + n_text
    log(f"  rope_apply grid={grid} n_text={n_text} heads={heads} dtype={dtype}")
    x = make_qkv(n, heads, 128, 77, dtype)
    q, _, _ = to_device(x)
    y = host_f64(fa.rope3d_apply(q, grid, n_text=n_text, rope_split=split))
    ref = oracle.rope3d_ref(x.q, grid, n_text, split)
    if dtype == "bf16":
        # one rounding of the fp32 result to bf16: |err| <= 2^-8 |ref| (+ fp32 noise)
        assert (np.abs(y - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()
    else:
        assert np.abs(y - ref).max() <= 3e-6
    # text rows pass through unchanged
    np.testing.assert_array_equal(y[T * H * W:], host_f64(q)[T * H * W:])
    # in place gives the same values
    y2 = host_f64(fa.rope3d_apply(q, grid, n_text=n_text, rope_split=split, out=q))
    np.testing.assert_array_equal(y2, y)


# ------------------------------------------------------------------------------------------
# Full attention, every element
# ------------------------------------------------------------------------------------------

def test_tiny_grid_f32():
    got, ref = run_full((3, 4, 6), 2, "f32", 0)
    assert_close(got, ref, "f32", "3x4x6 f32")


def test_tiny_grid_bf16():
    got, ref = run_full((3, 4, 6), 2, "bf16", 0)
    assert_close(got, ref, "bf16", "3x4x6 bf16")


@pytest.mark.parametrize("grid,n_text,heads,split", [
    ((1, 1, 1), 0, 1, WAN),          # a single token
    ((3, 5, 7), 0, 2, WAN),          # 105 rows: two key tiles, ragged
    ((7, 11, 13), 0, 2, WAN),        # 1,001 rows: four query tiles, ragged 41-key tail
    ((1, 16, 24), 0, 2, WAN),        # T' = 1
    ((37, 1, 1), 0, 2, WAN),         # H' = W' = 1
    ((2, 3, 4), 5, 3, WAN),          # text rows after a tiny grid
    ((1, 1, 1), 300, 2, WAN),        # (almost) text only
    ((5, 12, 13), 0, 2, HUN),        # HunyuanVideo split
    ((4, 16, 16), 0, 1, (0, 0, 128)),  # one axis carries every pair
    ((8, 8, 8), 64, 2, (128, 0, 0)),
])
def test_full_bf16_small(grid, n_text, heads, split):
    got, ref = run_full(grid, heads, "bf16", 100 + sum(grid) + n_text, n_text, split)
    assert_close(got, ref, "bf16", f"{grid}+{n_text}")


@pytest.mark.parametrize("grid,n_text,heads,split", [
    ((1, 1, 1), 0, 1, WAN), ((3, 5, 7), 0, 2, WAN), ((7, 11, 13), 0, 1, WAN),
    ((2, 3, 4), 5, 3, HUN), ((1, 1, 1), 70, 2, WAN),
])
def test_full_f32_small(grid, n_text, heads, split):
    got, ref = run_full(grid, heads, "f32", 200 + sum(grid) + n_text, n_text, split)
    assert_close(got, ref, "f32", f"{grid}+{n_text} f32")


def test_stress_value_offset_and_peaky_queries():
    # v + 10 exposes normalisation error as 10 dl / l.  Outputs near 10 are stored in bf16 with a
    # spacing of 2^-4, so the element bound adds the output rounding (2^-9 relative) to 2e-2;
    # relative L2 keeps the 5e-3 bar.  q x 8 makes the softmax peaky.
    got, ref = run_full((5, 9, 11), 2, "bf16", 300, v_offset=10.0)
    assert np.isfinite(got).all()
    _, rel = errors(got, ref)
    log(f"    v+10: rel_l2={rel:.3e}")
    assert rel <= 5e-3
    assert (np.abs(got - ref) <= 2e-2 + np.abs(ref) * 2.0 ** -9).all()
    got, ref = run_full((5, 9, 11), 2, "bf16", 301, q_mult=8.0)
    assert_close(got, ref, "bf16", "q*8")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_running_max_keeps_growing(dtype):
    # Peaky queries against keys whose norm grows along the sequence: every few tiles a row's
    # maximum moves past the stored one, so the rescale of the accumulator is taken many times.
    # Scores reach |s| ~ 100 in log2 units here, far outside the N(0,1) workloads the 2e-2 bound
    # is set for: fp16 rounding (2^-11) of rotated q and k moves such scores by up to ~0.05, which
    # moves near-tied weights by up to ~3 %, times value differences of up to ~6.  bf16 is held
    # to the relative-L2 bar and max-abs 5e-2.  In f32 the same scores carry ~100 x 2^-24 of
    # rounding in the exponent, so f32 keeps relative L2 <= 1e-5 and max-abs <= 1e-4.
    got, ref = run_full((4, 9, 10), 2, dtype, 305, q_mult=6.0, k_ramp=3.0)
    assert np.isfinite(got).all()
    max_abs, rel = errors(got, ref)
    log(f"    growing maximum {dtype}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert rel <= 1e-5 and max_abs <= 1e-4
    else:
        assert rel <= 5e-3 and max_abs <= 5e-2


# The attend step runs a fast kernel (16x16x32 blocks; score offset from each row's first 64 keys,
# never moved) and a guard launch that redoes, with the running-max kernel (32x32x16 blocks), every
# 256-row block whose row sums reached 2^64.  It does so from 32768 (block, 64-key tile) pairs up;
# 16384 tokens x 2 heads is the smallest grid of that size.  The partial-attention entry point runs
# the running-max kernel alone over the same rows.
FAST_GRID = (8, 32, 64)


def test_fast_launch_agrees_with_running_max_kernel():
    """N(0,1) inputs never move a row's maximum by more than 8 after the first tile, so the two
    kernels evaluate the same weights; they differ only in the order of their fp32 sums (and so
    in a few roundings of weights and outputs to bf16).  Each meets the parity bar against the
    oracle on sampled rows, and the two agree to a fifth of the relative-L2 bar everywhere."""
    n = 8 * 32 * 64
    log(f"  fast launch vs running-max kernel grid={FAST_GRID} heads=2 dtype=bf16 seed=330")
    x = make_qkv(n, 2, 128, 330, "bf16")
    q, k, v = to_device(x)
    fast = fa.attn3d(q, k, v, FAST_GRID)
    safe, _ = fa.attn3d_partial(q, k, v, FAST_GRID, q_begin=0, kv_begin=0)
    torch.cuda.synchronize()
    got_fast, got_safe = host_f64(fast), host_f64(safe)
    max_abs, rel = errors(got_fast, got_safe)
    same = float(np.mean(got_fast == got_safe))
    log(f"    fast vs running-max: max_abs={max_abs:.3e} rel_l2={rel:.3e} identical={same:.3f}")
    assert rel <= 1e-3 and max_abs <= 2e-3
    rows = sample_rows(n, n, 2048, 256, 330)
    ref = oracle.full_attention_ref(x.q, x.k, x.v, FAST_GRID, 0, WAN, 10000.0, rows=rows, heads=[0, 1])
    assert_close(got_fast[rows], ref, "bf16", "fast launch")
    assert_close(got_safe[rows], ref, "bf16", "running-max kernel")


@pytest.mark.parametrize("q_mult,k_ramp", [(2.0, 1.5), (6.0, 3.0)])
def test_fast_launch_redoes_blocks_whose_weights_grow(q_mult, k_ramp):
    """Keys whose norm grows along the sequence: later tiles score far above the first one, the
    fast launch flags those blocks (row sums past 2^64, or infinite) and the guard redoes them."""
    n = 8 * 32 * 64
    rows = sample_rows(n, n, 2048, 384, 331)
    got, ref = run_full(FAST_GRID, 2, "bf16", 331, rows=rows, q_mult=q_mult, k_ramp=k_ramp)
    assert np.isfinite(got).all()
    max_abs, rel = errors(got, ref)
    log(f"    fast launch, growing maximum q_mult={q_mult} k_ramp={k_ramp}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    # bounds as in test_running_max_keeps_growing (scores of |s| ~ 100 in log2 units)
    assert rel <= 5e-3 and max_abs <= 5e-2
    # and the same rows from the running-max kernel alone agree to the same bound
    x = make_qkv(n, 2, 128, 331, "bf16", q_mult=q_mult, k_ramp=k_ramp)
    q, k, v = to_device(x)
    safe, _ = fa.attn3d_partial(q, k, v, FAST_GRID, q_begin=0, kv_begin=0)
    torch.cuda.synchronize()
    m2, r2 = errors(got, host_f64(safe)[rows])
    log(f"    fast launch vs running-max kernel: max_abs={m2:.3e} rel_l2={r2:.3e}")
    assert r2 <= 5e-3 and m2 <= 5e-2


def test_stage_attend_matches_fwd_bitwise():
    grid, heads = (5, 9, 11), 2
    x = make_qkv(495, heads, 128, 400, "bf16")
    q, k, v = to_device(x)
    a = fa.attn3d(q, k, v, grid)
    ws = fa.attn3d_stage(k, grid)
    b = fa.attn3d_attend(q, v, grid, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("grid,n_text,heads,split", [
    ((3, 5, 7), 0, 2, WAN), ((7, 11, 13), 0, 2, WAN), ((2, 3, 4), 5, 3, HUN), ((1, 1, 1), 300, 2, WAN),
])
def test_fused_rope_path(grid, n_text, heads, split):
    # K rotated on every tile load instead of a staging pass: same numerics (fp16 rotated K),
    # so the outputs agree bit for bit with the staged path, and with the oracle to tolerance.
    T, H, W = grid
    n = T * H * W + n_text
    log(f"  fused rope grid={grid} n_text={n_text} heads={heads}")
    x = make_qkv(n, heads, 128, 450 + n, "bf16")
    q, k, v = to_device(x)
    a = fa.attn3d_fused(q, k, v, grid, n_text=n_text, rope_split=split)
    b = fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split)
    assert_close(host_f64(a), ref, "bf16", f"fused {grid}+{n_text}")


def test_deterministic():
    grid, heads = (7, 11, 13), 3
    x = make_qkv(1001, heads, 128, 401, "bf16")
    q, k, v = to_device(x)
    outs = [fa.attn3d(q, k, v, grid).view(torch.int16).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ------------------------------------------------------------------------------------------
# Factorised
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("grid,heads,split", [
    ((3, 4, 6), 2, WAN), ((5, 7, 9), 3, WAN), ((1, 5, 7), 2, WAN), ((9, 1, 1), 2, WAN),
    ((33, 3, 4), 2, HUN), ((40, 2, 3), 1, WAN), ((2, 16, 20), 2, WAN),
])
def test_factorized_small(dtype, grid, heads, split):
    T, H, W = grid
    log(f"  factorised grid={grid} heads={heads} dtype={dtype}")
    x = make_qkv(T * H * W, heads, 128, 500 + sum(grid), dtype)
    q, k, v = to_device(x)
    got = host_f64(fa.attn_factorized(q, k, v, grid, rope_split=split))
    ref = oracle.factorized_ref(x.q, x.k, x.v, grid, split)
    assert_close(got, ref, dtype, f"factorised {grid} {dtype}")


def test_factorized_one_frame_equals_full():
    grid = (1, 9, 13)
    x = make_qkv(117, 2, 128, 600, "bf16")
    q, k, v = to_device(x)
    a = host_f64(fa.attn_factorized(q, k, v, grid))
    b = host_f64(fa.attn3d(q, k, v, grid))
    # stage 2 has one key of weight 1: out = bf16(O_s), the same rounding as the full kernel
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------------------------------
# Configurations shaped like the pages' workloads (sampled rows, all keys)
# ------------------------------------------------------------------------------------------

def test_config_tiny_full_and_factorized_f32():
    grid = (3, 4, 6)
    x = make_qkv(72, 2, 128, 0, "f32")
    q, k, v = to_device(x)
    assert_close(host_f64(fa.attn3d(q, k, v, grid)), oracle.full_attention_ref(x.q, x.k, x.v, grid),
                 "f32", "config tiny full f32")
    assert_close(host_f64(fa.attn_factorized(q, k, v, grid)),
                 oracle.factorized_ref(x.q, x.k, x.v, grid), "f32", "config tiny factorised f32")


def test_config_wan13b_17f_all_rows_two_heads_and_sample():
    grid, heads = (5, 30, 52), 12
    got, ref = run_full(grid, heads, "bf16", 1000, head_subset=[0, 11])
    assert_close(got, ref, "bf16", "5x30x52 all rows, heads 0 and 11")
    rows = sample_rows(7800, 7800, 1560, 512, 1003)
    got, ref = run_full(grid, heads, "bf16", 1000, rows=rows)
    assert_close(got, ref, "bf16", "5x30x52 sampled rows, 12 heads")


def test_config_wan13b_81f_sampled():
    grid, heads = (21, 30, 52), 12
    rows = sample_rows(32760, 32760, 1560, 512, 2003)
    got, ref = run_full(grid, heads, "bf16", 2000, rows=rows)
    assert_close(got, ref, "bf16", "21x30x52 sampled rows")


def test_config_wan13b_81f_factorized_sampled():
    grid, heads = (21, 30, 52), 12
    x = make_qkv(32760, heads, 128, 2000, "bf16")
    q, k, v = to_device(x)
    got = host_f64(fa.attn_factorized(q, k, v, grid))
    rows = sample_rows(32760, 32760, 1560, 512, 2003)
    log("  factorised 21x30x52 sampled rows")
    ref = oracle.factorized_ref(x.q, x.k, x.v, grid, rows=rows)
    assert_close(got[rows], ref, "bf16", "21x30x52 factorised sampled")


def test_config_wan14b_720p_sampled():
    grid, heads = (21, 45, 80), 40
    rows = sample_rows(75600, 75600, 3600, 512, 3003)
    got, ref = run_full(grid, heads, "bf16", 3000, rows=rows, row_scale=(0.5, 2.0))
    assert_close(got, ref, "bf16", "21x45x80 sampled rows, row-scaled inputs")


def test_config_hunyuan_joint_sampled():
    grid, heads, n_text = (33, 45, 80), 24, 256
    n = 118800 + n_text
    rows = sample_rows(n, 118800, 3600, 512, 4003)
    got, ref = run_full(grid, heads, "bf16", 4000, n_text=n_text, split=HUN, rows=rows)
    assert_close(got, ref, "bf16", "33x45x80 + 256 text sampled rows")


def test_reference_image_tokens_sampled():
    """The Wan-14B 720p clip with 3 reference images of 4,096 tokens each concatenated into the
    sequence (joint attention): N = 75,600 + 12,288 = 87,888, the shape whose attention costs 35 %
    more than the clip alone.  The pages do not place these tokens in the grid, so they are
    appended rows without rotation, as text is.  5 heads: one GPU's share of 40 over 8."""
    grid, heads, n_text = (21, 45, 80), 5, 3 * 4096
    n = 75600 + n_text
    rows = sample_rows(n, 75600, 3600, 512, 5003)
    got, ref = run_full(grid, heads, "bf16", 5000, n_text=n_text, rows=rows)
    assert_close(got, ref, "bf16", "21x45x80 + 3 reference images (87,888 tokens) sampled rows")
