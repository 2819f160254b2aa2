"""Seeded random shapes through every attention entry point, against the float64 oracle.

The other GPU tests pick their shapes by hand, one for each edge a kernel was written for.  These
cases draw grids, head counts, text rows, RoPE splits, windows, key runs and projection widths
from fixed seeds, so that every entry point and launch choice also meets shapes nobody chose:
- the running-max kernel alone;
- the fast launch with its guard, with and without the key split and its merge;
- the window row map;
- the temporal kernels for T' up to 32, up to 64 and longer;
- the QKV projection, the merge of 1 to 16 key runs, the stand-alone rotation (other head sizes
  too) and the allocation-free entry (bit-identical to attn3d).

Each case's parameters follow from its seed alone (`case_*` below) and are printed before it runs.
The bar is the same as everywhere else: bf16 must meet max-abs 2e-2 and relative L2 5e-3 over the
compared elements, and the fp32 mode 1e-5.  Large cases compare a seeded sample of query rows per
head, edge rows included.  The partial-attention log-sum-exp is held to 1e-2 (bf16) and 1e-5 (fp32).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import full_spatiotemporal_attention_amd as fa
from full_spatiotemporal_attention_amd import _lib
from st_inputs import make_qkv, sample_rows, sample_rows_per_head
from parity_util import assert_close, host_f64, log, to_device

pytestmark = pytest.mark.gpu

WAN = (44, 42, 42)
HUN = (16, 56, 56)
LSE_TOL = {"bf16": 1e-2, "f32": 1e-5}
ROWS_PER_HEAD = 48


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()


# ---- case generators: plain functions of a seed -----------------------------------------------

def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _int(g, lo, hi):
    """Uniform integer in [lo, hi]."""
    return int(g.integers(lo, hi + 1))


def _split(g):
    """Wan's or HunyuanVideo's split, or a random one (even ranges summing to 128, zeros allowed)."""
    r = _int(g, 0, 3)
    if r == 0:
        return WAN
    if r == 1:
        return HUN
    dt = 2 * _int(g, 0, 64)
    dh = 2 * _int(g, 0, (128 - dt) // 2)
    return (dt, dh, 128 - dt - dh)


def _grid(g, max_tokens, t_range=(1, 12), h_max=40, w_max=70, min_tokens=1):
    while True:
        grid = (_int(g, *t_range), _int(g, 1, h_max), _int(g, 1, w_max))
        if min_tokens <= grid[0] * grid[1] * grid[2] <= max_tokens:
            return grid


def _heads(g, n, max_heads, max_rows_heads):
    return max(1, min(_int(g, 1, max_heads), max_rows_heads // n))


def case_full(seed):
    g = _rng(seed)
    grid = _grid(g, 40000)
    n_text = _int(g, 1, 300) if _int(g, 0, 2) == 1 else 0
    n = grid[0] * grid[1] * grid[2] + n_text
    return dict(grid=grid, n_text=n_text, heads=_heads(g, n, 6, 120000), split=_split(g),
                row_scale=(0.5, 2.0) if _int(g, 0, 3) == 0 else None)


def case_full_f32(seed):
    g = _rng(seed)
    grid = _grid(g, 1500, (1, 6), 20, 30)
    n_text = _int(g, 1, 100) if _int(g, 0, 1) else 0
    return dict(grid=grid, n_text=n_text, heads=_int(g, 1, 3), split=_split(g))


def case_factorized(seed, t_range):
    g = _rng(seed)
    grid = _grid(g, 60000, t_range, 45, 80)
    n = grid[0] * grid[1] * grid[2]
    return dict(grid=grid, heads=_heads(g, n, 6, 180000), split=_split(g))


def case_window(seed, large):
    """``large``: windows of 384 to 3,072 tokens, so that most such cases take the fast launch."""
    g = _rng(seed)
    while True:
        if large:
            window = (_int(g, 4, 8), _int(g, 8, 16), _int(g, 12, 24))
        else:
            window = (_int(g, 1, 8), _int(g, 1, 16), _int(g, 1, 24))
        counts = (_int(g, 1, 3), _int(g, 1, 3), _int(g, 1, 3))
        grid = tuple(w * c for w, c in zip(window, counts))
        if grid[0] * grid[1] * grid[2] <= 40000:
            break
    n = grid[0] * grid[1] * grid[2]
    heads = _heads(g, n, 12, 240000) if large else _heads(g, n, 6, 160000)
    return dict(grid=grid, window=window, heads=heads, split=_split(g))


def case_cross(seed):
    g = _rng(seed)
    n_q = _int(g, 1, 40000)
    return dict(n_q=n_q, n_kv=_int(g, 1, 1500), heads=_heads(g, n_q, 6, 120000))


def case_partial(seed, large):
    """``large``: grids of at least 12,000 tokens, so that long runs take the fast launch."""
    g = _rng(seed)
    grid = _grid(g, 30000, min_tokens=12000 if large else 1)
    n_text = _int(g, 1, 200) if _int(g, 0, 2) == 1 else 0
    n = grid[0] * grid[1] * grid[2] + n_text
    qb = _int(g, 0, n - 1)
    qc = _int(g, 1, min(n - qb, 3000))
    kb = _int(g, 0, n // 2)
    kc = n - kb if _int(g, 0, 1) else _int(g, 1, n - kb)   # half of the runs reach the last row
    heads = _heads(g, n, 8, 240000) if large else _heads(g, n, 6, 90000)
    return dict(grid=grid, n_text=n_text, heads=heads, split=_split(g),
                q_run=(qb, qc), kv_run=(kb, kc))


# ST_RANDOM_SHAPES_SCALE=k (default 2) runs k times the base count of cases per family: the base
# seeds, then seeds from base + 100000 on.  Larger k is a wider sweep.
SCALE = max(1, int(os.environ.get("ST_RANDOM_SHAPES_SCALE", "2")))


def _seeds(base, count):
    return list(range(base, base + count)) + list(range(base + 100000, base + 100000 + count * (SCALE - 1)))


FULL = [(s, case_full(s)) for s in _seeds(8100, 16)]
FULL_F32 = [(s, case_full_f32(s)) for s in _seeds(8150, 5)]
FACT = [(s, case_factorized(s, [(1, 32), (33, 64), (65, 90)][i % 3])) for i, s in enumerate(_seeds(8200, 9))]
WINDOW = [(s, case_window(s, s % 2 == 0)) for s in _seeds(8300, 8)]
CROSS = [(s, case_cross(s)) for s in _seeds(8400, 8)]
PARTIAL = [(s, case_partial(s, s % 2 == 0)) for s in _seeds(8500, 8)]


def _ids(cases):
    return [f"seed{s}" for s, _ in cases]


# ---- the cases ---------------------------------------------------------------------------------

@pytest.mark.parametrize("seed,c", FULL, ids=_ids(FULL))
def test_full_random(seed, c):
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    nv = grid[0] * grid[1] * grid[2]
    n = nv + n_text
    log(f"  attn3d seed={seed} grid={grid} n_text={n_text} heads={heads} split={split} "
        f"row_scale={c['row_scale']}")
    x = make_qkv(n, heads, 128, seed, "bf16", row_scale=c["row_scale"])
    q, k, v = to_device(x)
    out = fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    got = host_f64(out)
    gs, rs = [], []
    for hd in range(heads):
        rows = sample_rows_per_head(n, nv, grid[1] * grid[2], ROWS_PER_HEAD, seed + 17, hd)
        rs.append(oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0, rows=rows,
                                            heads=[hd]).ravel())
        gs.append(got[rows, hd].ravel())
    assert_close(np.concatenate(gs), np.concatenate(rs), "bf16", f"attn3d seed {seed}")


@pytest.mark.parametrize("seed,c", FULL_F32, ids=_ids(FULL_F32))
def test_full_f32_random(seed, c):
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  attn3d f32 seed={seed} grid={grid} n_text={n_text} heads={heads} split={split}")
    x = make_qkv(n, heads, 128, seed, "f32")
    q, k, v = to_device(x)
    out = fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0)
    assert_close(host_f64(out), ref, "f32", f"attn3d f32 seed {seed}")


@pytest.mark.parametrize("seed,c", FACT, ids=_ids(FACT))
def test_factorized_random(seed, c):
    grid, heads, split = c["grid"], c["heads"], c["split"]
    n = grid[0] * grid[1] * grid[2]
    log(f"  attn_factorized seed={seed} grid={grid} heads={heads} split={split}")
    x = make_qkv(n, heads, 128, seed, "bf16")
    q, k, v = to_device(x)
    out = fa.attn_factorized(q, k, v, grid, rope_split=split)
    torch.cuda.synchronize()
    rows = sample_rows(n, n, grid[1] * grid[2], ROWS_PER_HEAD, seed + 17)
    ref = oracle.factorized_ref(x.q, x.k, x.v, grid, split, 10000.0, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", f"attn_factorized seed {seed}")


@pytest.mark.parametrize("seed,c", WINDOW, ids=_ids(WINDOW))
def test_window_random(seed, c):
    grid, window, heads, split = c["grid"], c["window"], c["heads"], c["split"]
    n = grid[0] * grid[1] * grid[2]
    log(f"  attn_window seed={seed} grid={grid} window={window} heads={heads} split={split}")
    x = make_qkv(n, heads, 128, seed, "bf16")
    q, k, v = to_device(x)
    out = fa.attn_window(q, k, v, grid, window, rope_split=split)
    torch.cuda.synchronize()
    rows = sample_rows(n, n, grid[1] * grid[2], 4 * ROWS_PER_HEAD, seed + 17)
    ref = oracle.window_attention_ref(x.q, x.k, x.v, grid, window, split, 10000.0, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", f"attn_window seed {seed}")


@pytest.mark.parametrize("seed,c", CROSS, ids=_ids(CROSS))
def test_cross_random(seed, c):
    n_q, n_kv, heads = c["n_q"], c["n_kv"], c["heads"]
    log(f"  attn_cross seed={seed} n_q={n_q} n_kv={n_kv} heads={heads}")
    xq = make_qkv(n_q, heads, 128, seed, "bf16")
    xk = make_qkv(n_kv, heads, 128, seed + 10, "bf16")
    q = to_device(xq)[0]
    _, k, v = to_device(xk)
    out = fa.attn_cross(q, k, v)
    torch.cuda.synchronize()
    rows = sample_rows(n_q, n_q, n_q, 4 * ROWS_PER_HEAD, seed + 17)
    ref = oracle.cross_attention_ref(xq.q, xk.k, xk.v, rows=rows)
    assert_close(host_f64(out)[rows], ref, "bf16", f"attn_cross seed {seed}")


@pytest.mark.parametrize("seed,c", PARTIAL, ids=_ids(PARTIAL))
def test_partial_random(seed, c):
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    (qb, qc), (kb, kc) = c["q_run"], c["kv_run"]
    n = grid[0] * grid[1] * grid[2] + n_text
    log(f"  attn3d_partial seed={seed} grid={grid} n_text={n_text} heads={heads} split={split} "
        f"q=[{qb},+{qc}) kv=[{kb},+{kc})")
    x = make_qkv(n, heads, 128, seed, "bf16")
    q, k, v = to_device(x)
    o, lse = fa.attn3d_partial(q[qb:qb + qc].contiguous(), k[kb:kb + kc].contiguous(),
                               v[kb:kb + kc].contiguous(), grid, q_begin=qb, kv_begin=kb,
                               n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    got_o, got_l = host_f64(o), host_f64(lse)
    # The first and the last stretch of at most 128 query rows (one stretch if they overlap).
    stretches = sorted({(0, min(128, qc)), (max(0, qc - 128), qc)})
    for a, b in stretches:
        ro, rl = oracle.partial_attention_ref(x.q[qb + a:qb + b], x.k[kb:kb + kc], x.v[kb:kb + kc],
                                              grid, n_text, split, 10000.0, q_begin=qb + a,
                                              kv_begin=kb)
        assert_close(got_o[a:b], ro, "bf16", f"attn3d_partial seed {seed} rows [{a}, {b})")
        err = float(np.abs(got_l[a:b] - rl).max())
        log(f"    lse rows [{a}, {b}) max_abs={err:.3e}")
        assert err <= LSE_TOL["bf16"]


# ---- the entry points around the attention kernels ---------------------------------------------

def case_qkv(seed):
    g = _rng(seed)
    grid = _grid(g, 20000)
    n_text = _int(g, 1, 200) if _int(g, 0, 2) == 1 else 0
    return dict(grid=grid, n_text=n_text, heads=_int(g, 1, 10), split=_split(g),
                bias=bool(_int(g, 0, 3)))


def case_merge(seed):
    g = _rng(seed)
    grid = _grid(g, 3000, (1, 6), 20, 30)
    n_text = _int(g, 1, 60) if _int(g, 0, 2) == 1 else 0
    n = grid[0] * grid[1] * grid[2] + n_text
    n_runs = min(_int(g, 1, 16), n)
    cuts = sorted(set(int(c) for c in g.choice(np.arange(1, n), size=n_runs - 1, replace=False))) if n_runs > 1 else []
    return dict(grid=grid, n_text=n_text, heads=_int(g, 1, 3), split=_split(g), cuts=[0] + cuts + [n])


def case_rope(seed):
    g = _rng(seed)
    grid = _grid(g, 40000)
    n_text = _int(g, 1, 300) if _int(g, 0, 2) == 1 else 0
    if seed % 2 == 0:                            # another head size (bf16 serves d % 8 == 0)
        d = 8 * _int(g, 1, 32)
        dt = 2 * _int(g, 0, d // 2)
        dh = 2 * _int(g, 0, (d - dt) // 2)
        split = (dt, dh, d - dt - dh)
    else:
        split = _split(g)
    n = grid[0] * grid[1] * grid[2] + n_text
    return dict(grid=grid, n_text=n_text, heads=_heads(g, n, 12, 200000), split=split)


def case_noalloc(seed):
    g = _rng(seed)
    grid = _grid(g, 30000)
    n_text = _int(g, 1, 300) if _int(g, 0, 2) == 1 else 0
    n = grid[0] * grid[1] * grid[2] + n_text
    return dict(grid=grid, n_text=n_text, heads=_heads(g, n, 6, 90000), split=_split(g))


QKV = [(s, case_qkv(s)) for s in _seeds(8600, 6)]
MERGE = [(s, case_merge(s)) for s in _seeds(8700, 6)]
ROPE = [(s, case_rope(s)) for s in _seeds(8800, 6)]
NOALLOC = [(s, case_noalloc(s)) for s in _seeds(8900, 4)]


@pytest.mark.parametrize("seed,c", QKV, ids=_ids(QKV))
def test_qkv_rope_random(seed, c):
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    n = grid[0] * grid[1] * grid[2] + n_text
    ch = heads * 128
    log(f"  qkv_rope seed={seed} grid={grid} n_text={n_text} heads={heads} (C={ch}) split={split} "
        f"bias={c['bias']}")
    g = _rng(seed + 1)
    host = [make_bf16(g.standard_normal((n, ch))),
            make_bf16(g.standard_normal((3 * ch, ch)) / np.sqrt(ch)),
            make_bf16(0.1 * g.standard_normal(3 * ch)) if c["bias"] else None]
    x, w, b = (None if a is None else torch.from_numpy(a).to(torch.bfloat16).cuda() for a in host)
    q, k, v = fa.qkv_rope(x, w, grid, bias=b, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    rows = sample_rows(n, n - n_text, grid[1] * grid[2], 8 * ROWS_PER_HEAD, seed + 17)
    refs = oracle.qkv_rope_ref(host[0], host[1], host[2], grid, n_text, split, 10000.0, rows=rows)
    for name, got, ref in zip("qkv", (q, k, v), refs):
        assert_close(host_f64(got)[rows], ref, "bf16", f"qkv_rope seed {seed} {name}")


def make_bf16(a):
    """float64 values rounded once to bf16, returned as float32 (the exact bf16 values)."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("seed,c", MERGE, ids=_ids(MERGE))
def test_merge_random(seed, c):
    grid, n_text, heads, split, cuts = c["grid"], c["n_text"], c["heads"], c["split"], c["cuts"]
    log(f"  merge seed={seed} grid={grid} n_text={n_text} heads={heads} split={split} runs={len(cuts) - 1}")
    n = cuts[-1]
    x = make_qkv(n, heads, 128, seed, "bf16")
    q, k, v = to_device(x)
    parts = [fa.attn3d_partial(q, k[a:b].contiguous(), v[a:b].contiguous(), grid, q_begin=0,
                               kv_begin=a, n_text=n_text, rope_split=split)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = fa.attn_merge(parts)
    torch.cuda.synchronize()
    rows = sample_rows(n, n - n_text, grid[1] * grid[2], 4 * ROWS_PER_HEAD, seed + 17)
    ref = oracle.full_attention_ref(x.q, x.k, x.v, grid, n_text, split, 10000.0, rows=rows)
    assert_close(host_f64(o)[rows], ref, "bf16", f"merge of {len(cuts) - 1} runs, seed {seed}")
    _, rl = oracle.partial_attention_ref(x.q[rows[0]:rows[0] + 1], x.k, x.v, grid, n_text, split,
                                         10000.0, q_begin=int(rows[0]))
    err = float(np.abs(host_f64(lse)[rows[0]] - rl[0]).max())
    log(f"    merged lse (row {rows[0]}) max_abs={err:.3e}")
    assert err <= LSE_TOL["bf16"]


@pytest.mark.parametrize("seed,c", ROPE, ids=_ids(ROPE))
def test_rope_apply_random(seed, c):
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    d = sum(split)
    nv = grid[0] * grid[1] * grid[2]
    log(f"  rope3d_apply seed={seed} grid={grid} n_text={n_text} heads={heads} d={d} split={split}")
    x = make_qkv(nv + n_text, heads, d, seed, "bf16")
    q = to_device(x)[0]
    y = host_f64(fa.rope3d_apply(q, grid, n_text=n_text, rope_split=split))
    ref = oracle.rope3d_ref(x.q, grid, n_text, split)
    # one rounding of the rotated value to bf16: |err| <= 2^-8 |ref| (+ fp32 noise)
    bad = int((np.abs(y - ref) > np.abs(ref) * 2.0 ** -8 + 1e-6).sum())
    log(f"    elements past one bf16 rounding: {bad}")
    assert bad == 0
    np.testing.assert_array_equal(y[nv:], host_f64(q)[nv:])   # text rows pass through


@pytest.mark.parametrize("seed,c", NOALLOC, ids=_ids(NOALLOC))
def test_noalloc_random(seed, c):
    """The allocation-free entry against attn3d on the same inputs: the same launches on another
    workspace, so the outputs are identical bit for bit."""
    grid, n_text, heads, split = c["grid"], c["n_text"], c["heads"], c["split"]
    n = grid[0] * grid[1] * grid[2] + n_text
    limit = int(_lib.load().st_attn3d_noalloc_scratch_bytes())
    while heads > 1 and fa.attn3d_workspace_bytes(grid, heads, n_text, 128, split) > limit:
        heads -= 1
    log(f"  attn3d_noalloc seed={seed} grid={grid} n_text={n_text} heads={heads} split={split}")
    q, k, v = to_device(make_qkv(n, heads, 128, seed, "bf16"))
    a = fa.attn3d_noalloc(q, k, v, grid, n_text=n_text, rope_split=split)
    b = fa.attn3d(q, k, v, grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
