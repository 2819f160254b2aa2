"""GPU parity for the rows next to the hot path: text cross-attention, partial attention over a
run of keys (with its log-sum-exp), and the merge of partials, against the float64 oracle.

All calls go through the C ABI of libstattn.so.  Tolerances as in test_gpu_parity; the log-sum-exp
of the bf16 path (scores from fp16-rounded rotated q and k) is checked to 1e-2 absolute, that of
the fp32 mode to 1e-5.
"""
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
LSE_TOL = {"bf16": 1e-2, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()


def qkv_pair(n_q, n_kv, heads, dtype, seed):
    """Queries from one seeded set, keys/values from another (different row counts)."""
    xq = make_qkv(n_q, heads, 128, seed, dtype)
    xk = make_qkv(n_kv, heads, 128, seed + 10, dtype)
    q = to_device(xq)[0]
    _, k, v = to_device(xk)
    return xq.q, xk.k, xk.v, q, k, v


# ---- text cross-attention -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_q,n_kv,heads", [(1000, 77, 3), (300, 512, 2), (1, 1, 1), (257, 64, 2),
                                            (64, 129, 1)])
def test_cross_attention(dtype, n_q, n_kv, heads):
    log(f"  cross n_q={n_q} n_kv={n_kv} heads={heads} dtype={dtype} seed=7100")
    qh, kh, vh, q, k, v = qkv_pair(n_q, n_kv, heads, dtype, 7100)
    out = fa.attn_cross(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.cross_attention_ref(qh, kh, vh)
    assert_close(host_f64(out), ref, dtype, f"cross {n_q}x{n_kv} {dtype}")


def test_cross_attention_wan_text_sampled():
    """Wan-shaped: 21x30x52 = 32,760 video queries against 512 text tokens, 12 heads."""
    n_q, n_kv, heads = 32760, 512, 12
    log(f"  cross n_q={n_q} n_kv={n_kv} heads={heads} dtype=bf16 seed=7200 rows=512")
    qh, kh, vh, q, k, v = qkv_pair(n_q, n_kv, heads, "bf16", 7200)
    out = fa.attn_cross(q, k, v)
    torch.cuda.synchronize()
    rows = sample_rows(n_q, n_q, 1560, 512, 7203)
    ref = oracle.cross_attention_ref(qh, kh, vh, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", "cross 32760x512 sampled")


def test_cross_attention_fast_launch_ragged():
    """20,000 queries (the last query tile holds 32 rows) against 300 text keys (the last key tile
    holds 44), 12 heads: 79 x 12 items of 5 key tiles take the fast launch.  Sampled rows plus the
    whole short tile against the oracle."""
    n_q, n_kv, heads = 20000, 300, 12
    log(f"  cross n_q={n_q} n_kv={n_kv} heads={heads} dtype=bf16 seed=7250 (fast launch, ragged)")
    qh, kh, vh, q, k, v = qkv_pair(n_q, n_kv, heads, "bf16", 7250)
    out = fa.attn_cross(q, k, v)
    torch.cuda.synchronize()
    rows = np.union1d(sample_rows(n_q, n_q, 1560, 512, 7253), np.arange(19968, n_q))
    ref = oracle.cross_attention_ref(qh, kh, vh, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", "cross 20000x300 fast launch")


# ---- partial attention and merge ---------------------------------------------------------------

def grid_inputs(grid, n_text, heads, dtype, seed, split):
    n = grid[0] * grid[1] * grid[2] + n_text
    x = make_qkv(n, heads, 128, seed, dtype)
    return x, to_device(x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid,n_text,split,qb,qc,kb,kc", [
    ((5, 6, 7), 9, WAN, 17, 100, 40, 90),
    ((3, 8, 8), 0, HUN, 0, 192, 100, 92),
    ((2, 5, 5), 4, WAN, 50, 4, 0, 1),
])
def test_partial_matches_oracle(dtype, grid, n_text, split, qb, qc, kb, kc):
    log(f"  partial grid={grid} n_text={n_text} q=[{qb},+{qc}) kv=[{kb},+{kc}) dtype={dtype} seed=7300")
    x, (q, k, v) = grid_inputs(grid, n_text, 2, dtype, 7300, split)
    o, lse = fa.attn3d_partial(q[qb:qb + qc].contiguous(), k[kb:kb + kc].contiguous(),
                               v[kb:kb + kc].contiguous(), grid, q_begin=qb, kv_begin=kb,
                               n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    ro, rl = oracle.partial_attention_ref(x.q[qb:qb + qc], x.k[kb:kb + kc], x.v[kb:kb + kc], grid,
                                          n_text, split, 10000.0, q_begin=qb, kv_begin=kb)
    assert_close(host_f64(o), ro, dtype, f"partial o {dtype}")
    err = float(np.abs(host_f64(lse) - rl).max())
    log(f"    partial lse max_abs={err:.3e}")
    assert err <= LSE_TOL[dtype]


def test_partial_fast_launch_with_lse():
    """1,000 query rows (the last 256-row block holds 232) against a run of 8,192 keys of the
    21x30x52 grid, 8 heads: 4 blocks x 8 heads x 128 key tiles take the fast launch, which writes
    the log-sum-exp itself.  Two stretches of rows (the first block's start, the short block)
    against the oracle, output and log-sum-exp."""
    grid, heads = (21, 30, 52), 8
    qb, qc, kb, kc = 12000, 1000, 4000, 8192
    log(f"  partial (fast launch) grid={grid} heads={heads} q=[{qb},+{qc}) kv=[{kb},+{kc}) seed=7350")
    x, (q, k, v) = grid_inputs(grid, 0, heads, "bf16", 7350, WAN)
    o, lse = fa.attn3d_partial(q[qb:qb + qc].contiguous(), k[kb:kb + kc].contiguous(),
                               v[kb:kb + kc].contiguous(), grid, q_begin=qb, kv_begin=kb)
    torch.cuda.synchronize()
    got_o, got_l = host_f64(o), host_f64(lse)
    for a, b in ((0, 128), (872, 1000)):
        ro, rl = oracle.partial_attention_ref(x.q[qb + a:qb + b], x.k[kb:kb + kc], x.v[kb:kb + kc], grid,
                                              0, WAN, 10000.0, q_begin=qb + a, kv_begin=kb)
        assert_close(got_o[a:b], ro, "bf16", f"partial fast launch o rows [{a}, {b})")
        err = float(np.abs(got_l[a:b] - rl).max())
        log(f"    partial fast launch lse rows [{a}, {b}) max_abs={err:.3e}")
        assert err <= LSE_TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_of_key_runs_equals_full_attention(dtype):
    grid, n_text, split, heads = (4, 9, 10), 20, WAN, 2
    n = grid[0] * grid[1] * grid[2] + n_text
    cuts = [0, 100, 101, 230, n]
    log(f"  merge grid={grid} n_text={n_text} runs={cuts} dtype={dtype} seed=7400")
    x, (q, k, v) = grid_inputs(grid, n_text, heads, dtype, 7400, split)
    parts = [fa.attn3d_partial(q, k[a:b].contiguous(), v[a:b].contiguous(), grid, q_begin=0,
                               kv_begin=a, n_text=n_text, rope_split=split)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = fa.attn_merge(parts)
    torch.cuda.synchronize()
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0)
    assert_close(host_f64(o), ref, dtype, f"merge of 4 runs {dtype}")
    _, rl = oracle.partial_attention_ref(x.q, x.k, x.v, grid, n_text, split)
    err = float(np.abs(host_f64(lse) - rl).max())
    log(f"    merged lse max_abs={err:.3e}")
    assert err <= LSE_TOL[dtype]
    # the merge kernel alone, on the GPU's own partials, against the oracle's merge of them
    ro, rl2 = oracle.merge_partials_ref([(host_f64(a), host_f64(b)) for a, b in parts])
    m_abs, m_rel = errors(host_f64(o), ro)
    log(f"    merge kernel vs oracle merge of the same partials: max_abs={m_abs:.3e} rel_l2={m_rel:.3e}")
    if dtype == "f32":
        assert m_abs <= 1e-6
    else:
        assert m_abs <= 2 ** -8 * float(np.abs(ro).max()) + 1e-6   # one bf16 rounding of the output
    assert float(np.abs(host_f64(lse) - rl2).max()) <= 1e-5


@pytest.mark.parametrize("n_runs", [3, 5, 8])
def test_merge_part_counts(n_runs):
    # 2, 3 and 4 parts have kernels of their own; other counts take the general kernel.
    grid, n_text, split, heads = (3, 5, 7), 6, WAN, 2
    n = grid[0] * grid[1] * grid[2] + n_text
    cuts = [round(i * n / n_runs) for i in range(n_runs)] + [n]
    log(f"  merge of {n_runs} runs grid={grid} n_text={n_text} cuts={cuts} seed={7600 + n_runs}")
    x, (q, k, v) = grid_inputs(grid, n_text, heads, "bf16", 7600 + n_runs, split)
    parts = [fa.attn3d_partial(q, k[a:b].contiguous(), v[a:b].contiguous(), grid, q_begin=0,
                               kv_begin=a, n_text=n_text, rope_split=split)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = fa.attn_merge(parts)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_partials_ref([(host_f64(a), host_f64(b)) for a, b in parts])
    m_abs, m_rel = errors(host_f64(o), ro)
    log(f"    merge vs oracle merge of the same partials: max_abs={m_abs:.3e} rel_l2={m_rel:.3e}")
    assert m_abs <= 2 ** -8 * float(np.abs(ro).max()) + 1e-6   # one bf16 rounding of the output
    assert float(np.abs(host_f64(lse) - rl).max()) <= 1e-5
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0)
    assert_close(host_f64(o), ref, "bf16", f"merge of {n_runs} runs")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_in_place_and_single_part(dtype):
    grid, split, heads = (3, 6, 6), WAN, 3
    n = grid[0] * grid[1] * grid[2]
    log(f"  merge in place grid={grid} dtype={dtype} seed=7500")
    x, (q, k, v) = grid_inputs(grid, 0, heads, dtype, 7500, split)
    parts = [fa.attn3d_partial(q, k[a:b].contiguous(), v[a:b].contiguous(), grid, kv_begin=a,
                               rope_split=split) for a, b in [(0, 40), (40, n)]]
    o_ref, l_ref = fa.attn_merge(parts)
    o0, l0 = parts[0][0].clone(), parts[0][1].clone()
    o_one, l_one = fa.attn_merge([(o0, l0)])
    o_in, l_in = fa.attn_merge(parts, out=parts[0][0], lse_out=parts[0][1])
    torch.cuda.synchronize()
    assert o_in.data_ptr() == parts[0][0].data_ptr()
    assert torch.equal(o_in, o_ref) and torch.equal(l_in, l_ref)
    assert float((o_one.float() - o0.float()).abs().max()) <= (2 ** -8 if dtype == "bf16" else 1e-6)
    assert float((l_one - l0).abs().max()) <= 1e-6


# ---- QKV projection with the rotation of q and k ---------------------------------------------------

def qkv_inputs(n, heads, dtype, seed, with_bias=True):
    """x ~ N(0,1) [n, C], w ~ N(0, 1/C) [3C, C], bias ~ N(0, 0.1^2); bf16 inputs rounded once."""
    from st_inputs import f32_to_bf16_bits, bf16_bits_to_f32
    c = heads * 128
    rng = np.random.default_rng(seed)
    arrs = [rng.standard_normal((n, c)).astype(np.float32),
            (rng.standard_normal((3 * c, c)) / np.sqrt(c)).astype(np.float32),
            (0.1 * rng.standard_normal(3 * c)).astype(np.float32)]
    if dtype == "bf16":
        bits = [f32_to_bf16_bits(a) for a in arrs]
        host = [bf16_bits_to_f32(b) for b in bits]
        dev = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda() for b in bits]
    else:
        host = arrs
        dev = [torch.from_numpy(a).cuda() for a in arrs]
    if not with_bias:
        host[2], dev[2] = None, None
    return host, dev


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid,n_text,heads,split,bias", [
    ((3, 5, 7), 9, 2, WAN, True),
    ((2, 16, 20), 0, 3, HUN, True),      # 3C = 1152: a partial feature tile
    ((1, 1, 1), 0, 1, WAN, False),
])
def test_qkv_rope_small(dtype, grid, n_text, heads, split, bias):
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  qkv_rope grid={grid} n_text={n_text} heads={heads} split={split} bias={bias} dtype={dtype} seed=7600")
    (xh, wh, bh), (x, w, b) = qkv_inputs(n, heads, dtype, 7600, bias)
    q, k, v = fa.qkv_rope(x, w, grid, bias=b, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_ref(xh, wh, bh, grid, n_text, split)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(host_f64(got), ref, dtype, f"qkv_rope {name} {dtype}")


def test_qkv_rope_wan13b_sampled():
    """Wan2.1-1.3B-shaped projection: 32,760 tokens x 1,536 features -> 4,608, sampled rows."""
    grid, heads = (21, 30, 52), 12
    n = grid[0] * grid[1] * grid[2]
    log(f"  qkv_rope grid={grid} heads={heads} dtype=bf16 seed=7700 rows=512")
    (xh, wh, bh), (x, w, b) = qkv_inputs(n, heads, "bf16", 7700)
    q, k, v = fa.qkv_rope(x, w, grid, bias=b, rope_split=WAN)
    torch.cuda.synchronize()
    rows = sample_rows(n, n, 1560, 512, 7703)
    rq, rk, rv = oracle.qkv_rope_ref(xh, wh, bh, grid, 0, WAN, rows=rows)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(host_f64(got)[rows], ref, "bf16", f"qkv_rope 32760x1536 {name} sampled")


def test_qkv_rope_then_attention_equals_full_3d_attention():
    """Rotated q, k from the projection, then attention without rotation, against the oracle's
    3D-RoPE attention of the projected (unrotated) x w^T."""
    grid, n_text, heads, split = (3, 6, 8), 5, 2, WAN
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  qkv_rope + attention grid={grid} n_text={n_text} heads={heads} seed=7800")
    (xh, wh, _), (x, w, _) = qkv_inputs(n, heads, "bf16", 7800, with_bias=False)
    q, k, v = fa.qkv_rope(x, w, grid, n_text=n_text, rope_split=split)
    out = fa.attn_cross(q, k, v)
    torch.cuda.synchronize()
    c = heads * 128
    y = np.asarray(xh, np.float64) @ np.asarray(wh, np.float64).T
    ref = oracle.full_attention_ref(y[:, :c].reshape(n, heads, 128), y[:, c:2 * c].reshape(n, heads, 128),
                                    y[:, 2 * c:].reshape(n, heads, 128), grid, n_text, split)
    assert_close(host_f64(out), ref, "bf16", "qkv_rope then attention")


# ---- local 3D-window attention ------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid,window,split,heads", [
    ((4, 6, 8), (2, 3, 4), WAN, 2),        # 24 tokens per window: one partial key tile
    ((6, 10, 12), (3, 5, 6), HUN, 2),      # 90: a full tile and a ragged one
    ((4, 16, 16), (2, 8, 16), WAN, 1),     # 256: exactly one query block
    ((2, 9, 35), (1, 9, 35), WAN, 2),      # 315: the per-frame (spatial) case, two query blocks
    ((3, 8, 12), (3, 8, 12), HUN, 2),      # one window over the whole grid
])
def test_window_matches_oracle(dtype, grid, window, split, heads):
    log(f"  window grid={grid} window={window} split={split} heads={heads} dtype={dtype} seed=7600")
    x, (q, k, v) = grid_inputs(grid, 0, heads, dtype, 7600, split)
    out = fa.attn_window(q, k, v, grid, window, rope_split=split)
    torch.cuda.synchronize()
    ref = oracle.window_attention_ref(x.q, x.k, x.v, grid, window, split)
    assert_close(host_f64(out), ref, dtype, f"window {grid}/{window} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_of_one_token_returns_v(dtype):
    """Each token alone in its window: its only weight is exp(0) = 1, so out == v exactly."""
    grid = (3, 5, 7)
    log(f"  window grid={grid} window=(1,1,1) dtype={dtype} seed=7610")
    x, (q, k, v) = grid_inputs(grid, 0, 2, dtype, 7610, WAN)
    out = fa.attn_window(q, k, v, grid, (1, 1, 1))
    torch.cuda.synchronize()
    assert torch.equal(out, v)


def test_window_over_whole_grid_is_full_attention_bitwise():
    """With one window the row map is the identity and the kernel does the full path's arithmetic."""
    grid = (3, 10, 13)
    log(f"  window grid={grid} window=grid vs attn3d dtype=bf16 seed=7620")
    _, (q, k, v) = grid_inputs(grid, 0, 3, "bf16", 7620, WAN)
    a = fa.attn_window(q, k, v, grid, grid)
    b = fa.attn3d(q, k, v, grid)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_window_wan_grid_sampled():
    """21x30x52 grid (Wan 2.1, 81 frames at 480x832), 12 heads, windows of 7x10x13 = 910 tokens."""
    grid, window, heads = (21, 30, 52), (7, 10, 13), 12
    n = 32760
    log(f"  window grid={grid} window={window} heads={heads} dtype=bf16 seed=7630 rows=512")
    x, (q, k, v) = grid_inputs(grid, 0, heads, "bf16", 7630, WAN)
    out = fa.attn_window(q, k, v, grid, window)
    torch.cuda.synchronize()
    rows = sample_rows(n, n, 1560, 512, 7633)
    ref = oracle.window_attention_ref(x.q, x.k, x.v, grid, window, WAN, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", "window 21x30x52 / 7x10x13 sampled")


# Windows large enough that the attend step takes the fast launch (at least 32768 pairs of a
# 256-row block and a 64-key tile), so the 16x16x32 kernel's window row map runs as well.
def test_window_fast_launch_ragged_sampled():
    """4 windows of 7x15x26 = 2730 tokens (a partial last key tile, and a last query block whose
    last two waves have no rows), 20 heads: 4 x 11 blocks x 20 heads x 43 key tiles = 37840."""
    grid, window, heads = (7, 30, 52), (7, 15, 26), 20
    n = 7 * 30 * 52
    log(f"  window grid={grid} window={window} heads={heads} dtype=bf16 seed=7640 rows=384")
    x, (q, k, v) = grid_inputs(grid, 0, heads, "bf16", 7640, WAN)
    out = fa.attn_window(q, k, v, grid, window)
    torch.cuda.synchronize()
    rows = sample_rows(n, n, 1560, 384, 7641)
    ref = oracle.window_attention_ref(x.q, x.k, x.v, grid, window, WAN, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", "window 7x30x52 / 7x15x26, fast launch, sampled")


def test_window_over_whole_grid_fast_launch_bitwise():
    """One window over a 16,384-token grid, 4 heads (64 blocks x 4 heads x 256 key tiles): both
    calls take the fast launch (256 items, one per CU, so full attention does not split its keys),
    and with the identity row map they agree bit for bit."""
    grid = (8, 32, 64)
    log(f"  window grid={grid} window=grid vs attn3d (fast launch) dtype=bf16 seed=7650")
    _, (q, k, v) = grid_inputs(grid, 0, 4, "bf16", 7650, WAN)
    a = fa.attn_window(q, k, v, grid, grid)
    b = fa.attn3d(q, k, v, grid)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
