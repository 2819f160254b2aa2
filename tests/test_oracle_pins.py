"""Pins for the CPU oracle: printed values, closed forms, invariants, special cases, brute force.

Each check ties the oracle to something other than itself: numbers printed on the pages (the
fixtures under tests/golden cite them), an independent construction of the same mathematical
object (a matrix exponential, complex multiplication, torch's scaled_dot_product_attention), or a
special case whose answer is known in closed form.  The last group plants mistakes in copies of the
oracle and checks that at least one pin catches each.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import st_oracle as so
from st_inputs import make_qkv
from conftest import read_golden


# ------------------------------------------------------------------------------------------
# Shapes and costs against printed tables
# ------------------------------------------------------------------------------------------

def check_token_table(grid_fn):
    for row in read_golden("token_grids.txt"):
        _, frames, h, w, lt, lh, lw, tt, th, tw, n, dim, mult = row
        lat, grid, tokens, tdim = grid_fn(int(frames), int(h), int(w))
        assert lat == (int(lt), int(lh), int(lw))
        assert grid == (int(tt), int(th), int(tw))
        assert tokens == int(n)
        assert tdim == int(dim)
        assert round(tokens / 4096) == int(mult)


def test_token_grid_table():
    check_token_table(oracle.latent_token_grid)


def test_token_grid_closed_form_4k_plus_1():
    # T' = 1 + (T - 1)/4 exactly for frame counts of the form 4k + 1.
    for k in range(0, 40):
        lat, grid, _, _ = oracle.latent_token_grid(4 * k + 1, 480, 832)
        assert lat[0] == k + 1 and grid[0] == k + 1
    # The 17-frame 832x480 clip: 5 x 30 x 52 = 7,800 tokens.
    assert oracle.latent_token_grid(17, 480, 832)[1:3] == ((5, 30, 52), 7800)


def check_flop_table(model_fn):
    for row in read_golden("attn_flops.txt"):
        _, frames, h, w, hidden, layers, fact_t, full_t, ratio, lin_t = row
        _, grid, _, _ = oracle.latent_token_grid(int(frames), int(h), int(w))
        r = model_fn(grid, int(hidden), int(layers))
        assert round(r["factorized"] / 1e12) == int(fact_t)
        assert round(r["full"] / 1e12) == int(full_t)
        assert round(r["full"] / r["factorized"]) == int(ratio)
        assert round(r["linear"] / 1e12) == int(lin_t)


def test_attention_flop_table():
    check_flop_table(oracle.attn_flop_model)


def test_metric_flops_match_cost_model_per_head():
    # 4 N^2 D with D = heads * d is the page's full-attention cost for one layer.
    for grid, heads in [((21, 30, 52), 12), ((21, 45, 80), 40), ((3, 4, 6), 2)]:
        n = grid[0] * grid[1] * grid[2]
        assert oracle.metric_flops(n, heads, 128) == oracle.attn_flop_model(grid, heads * 128)["full"]
        assert oracle.factorized_flops(grid, heads, 128) == \
            oracle.attn_flop_model(grid, heads * 128)["factorized"]
    # One Wan2.1-14B layer at 720p / 81 frames: 4,682 TFLOP over 40 layers.
    assert oracle.metric_flops(75600, 40, 128) / 1e12 == pytest.approx(117.05, abs=0.01)


def test_worked_arithmetic():
    g = {r[0]: float(r[1]) for r in read_golden("worked_arithmetic.txt")}
    pixels = 81 * 832 * 480
    assert pixels == g["pixels_81f_832x480"]
    _, grid, n480, _ = oracle.latent_token_grid(81, 480, 832)
    assert round(2 * pixels ** 2 / 1e12) == g["raw_attention_TB_one_head"]
    assert round(pixels ** 2 / n480 ** 2) == g["attention_reduction"]
    assert round(3 * pixels / 1e6, 2) == g["pixel_floats_M"]
    lat, _, _, _ = oracle.latent_token_grid(81, 480, 832)
    assert round(16 * lat[0] * lat[1] * lat[2] / 1e6, 2) == g["latent_floats_M"]
    assert round(2 * n480 ** 2 / 1e9, 2) == g["token_scores_GB"]
    _, grid720, n720, _ = oracle.latent_token_grid(81, 720, 1280)
    assert round(n720 / n480, 1) == g["tokens_growth"]
    a480 = oracle.attn_flop_model(grid, 5120)["full"]
    a720 = oracle.attn_flop_model(grid720, 5120)["full"]
    assert round(a720 / a480, 1) == g["attention_growth"]
    l480 = oracle.attn_flop_model(grid, 5120)["linear"]
    l720 = oracle.attn_flop_model(grid720, 5120)["linear"]
    assert round(l720 / l480, 1) == g["linear_growth"]
    assert n720 + 3 * 4096 == g["tokens_with_refs"]
    assert round(100 * ((n720 + 3 * 4096) ** 2 / n720 ** 2 - 1)) == g["attention_increase_pct"]
    # Minimal DiT: latent [B, T', C, H', W'] = (1, 3, 4, 8, 8), patch 2 -> 3 x 4 x 4 tokens.
    t, h, w, vid = oracle.token_positions((3, 8 // 2, 8 // 2), n_text=4)
    assert vid.sum() == g["minimal_dit_video_tokens"] and t.size == g["minimal_dit_sequence"]
    r = oracle.attn_flop_model(grid720, 5120)
    assert round(r["full"] / r["factorized"] / 10) * 10 == g["wan720_full_over_factorized"]


def test_factorized_ratio_about_t_times():
    # Self-test answer 2: full costs about T' times factorised.  Closed form T'S / (S + T').
    for grid in [(21, 45, 80), (21, 30, 52), (3, 4, 6), (13, 30, 45)]:
        t, s = grid[0], grid[1] * grid[2]
        r = oracle.metric_flops(t * s, 1, 128) / oracle.factorized_flops(grid, 1, 128)
        assert r == pytest.approx(t * s / (s + t), rel=1e-12)
        if s >= 100 * t:
            assert r == pytest.approx(t, rel=0.01)


# ------------------------------------------------------------------------------------------
# Flat order
# ------------------------------------------------------------------------------------------

def check_shards(positions_fn):
    t, h, w, _ = positions_fn((2, 2, 3), 0)
    coords = list(zip(t.tolist(), h.tolist(), w.tolist()))
    shards = [coords[r * 12 // 3:(r + 1) * 12 // 3] for r in range(3)]
    for row in read_golden("shards.txt"):
        card = int(row[0])
        want = [tuple(int(c) for c in x.split(",")) for x in row[1:]]
        assert shards[card] == want


def test_flat_order_matches_printed_shards():
    check_shards(oracle.token_positions)


def test_flat_order_closed_form():
    t, h, w, vid = oracle.token_positions((5, 7, 11), n_text=3)
    n = np.arange(5 * 7 * 11)
    assert (t[:n.size] == n // 77).all() and (h[:n.size] == (n // 11) % 7).all()
    assert (w[:n.size] == n % 11).all()
    assert vid[:n.size].all() and not vid[n.size:].any()


# ------------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------------

def test_pair_counts():
    for row in read_golden("rope_splits.txt"):
        split = tuple(int(x) for x in row[1:4])
        pairs = [int(x) for x in row[4:7]]
        assert sum(split) == int(row[7])
        layout = oracle.rope_pair_layout(split)
        for axis in range(3):
            assert sum(1 for a, _, _ in layout if a == axis) == pairs[axis]
        assert len(oracle.rope_frequencies(split)[0]) == pairs[0]


def _r3d_matrix(pos, split, theta):
    """Explicit block-diagonal R_3D(t, y, x): one 2x2 rotation per pair, built as the matrix
    exponential of the rotation generator, then assembled with scipy's block_diag."""
    gen = np.array([[0.0, -1.0], [1.0, 0.0]])
    blocks = []
    freqs = oracle.rope_frequencies(split, theta)
    for axis, da in enumerate(split):
        for j in range(da // 2):
            blocks.append(scipy.linalg.expm(pos[axis] * freqs[axis][j] * gen))
    return scipy.linalg.block_diag(*blocks)


def check_rope_against_matrix(rope_fn):
    grid, split, theta = (4, 5, 7), (44, 42, 42), 10000.0
    x = np.random.default_rng(1).standard_normal((140, 2, 128))
    y = rope_fn(x, grid, 0, split, theta)
    t, h, w, _ = oracle.token_positions(grid)
    for n in [0, 1, 6, 7, 34, 35, 36, 71, 139]:
        r = _r3d_matrix((t[n], h[n], w[n]), split, theta)
        np.testing.assert_allclose(y[n], x[n] @ r.T, rtol=0, atol=1e-12)


def test_rope_equals_block_diagonal_matrix():
    check_rope_against_matrix(oracle.rope3d_ref)


def test_rope_hunyuan_split_matrix():
    grid, split = (3, 4, 6), (16, 56, 56)
    x = np.random.default_rng(2).standard_normal((72, 1, 128))
    y = oracle.rope3d_ref(x, grid, 0, split)
    t, h, w, _ = oracle.token_positions(grid)
    for n in [5, 23, 24, 71]:
        r = _r3d_matrix((t[n], h[n], w[n]), split, 10000.0)
        np.testing.assert_allclose(y[n, 0], r @ x[n, 0], rtol=0, atol=1e-12)


def test_rope_complex_form():
    # A 2-channel pair rotated by phi is the complex number x0 + i x1 times e^{i phi}.
    grid, split = (3, 4, 6), (44, 42, 42)
    x = np.random.default_rng(3).standard_normal((72, 1, 128))
    y = oracle.rope3d_ref(x, grid, 0, split)
    t, h, w, _ = oracle.token_positions(grid)
    freqs = oracle.rope_frequencies(split)
    off = 0
    for axis, da in enumerate(split):
        pos = (t, h, w)[axis]
        for j in range(da // 2):
            z = x[:, 0, off + 2 * j] + 1j * x[:, 0, off + 2 * j + 1]
            zr = z * np.exp(1j * pos * freqs[axis][j])
            np.testing.assert_allclose(y[:, 0, off + 2 * j], zr.real, atol=1e-12)
            np.testing.assert_allclose(y[:, 0, off + 2 * j + 1], zr.imag, atol=1e-12)
        off += da


def test_rope_norm_preserving():
    x = np.random.default_rng(4).standard_normal((21 * 5 * 6, 3, 128))
    y = oracle.rope3d_ref(x, (21, 5, 6), 0, (44, 42, 42))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def check_relative_invariance(rope_fn):
    # Same q and k vectors placed at (p_i, p_j) and at (p_i + D, p_j + D): equal scores.
    grid = (6, 7, 9)
    rng = np.random.default_rng(5)
    qv, kv = rng.standard_normal(128), rng.standard_normal(128)
    n_of = lambda t, h, w: (t * grid[1] + h) * grid[2] + w
    x = np.zeros((grid[0] * grid[1] * grid[2], 1, 128))
    cases = [((0, 0, 0), (2, 3, 4), (1, 1, 1)), ((1, 2, 3), (4, 0, 8), (1, 3, 0)),
             ((5, 6, 0), (0, 0, 8), (0, 0, 0)), ((2, 1, 5), (2, 4, 1), (3, 2, 3))]
    for pi, pj, dd in cases:
        s = []
        for shift in [(0, 0, 0), dd]:
            a = tuple(p + q for p, q in zip(pi, shift))
            b = tuple(p + q for p, q in zip(pj, shift))
            ia, ib = n_of(*a), n_of(*b)
            xq = x.copy(); xq[ia, 0] = qv
            xk = x.copy(); xk[ib, 0] = kv
            s.append(rope_fn(xq, grid, 0, (44, 42, 42), 10000.0)[ia, 0] @
                     rope_fn(xk, grid, 0, (44, 42, 42), 10000.0)[ib, 0])
        assert s[0] == pytest.approx(s[1], abs=1e-11)


def test_rope_relative_position_invariance():
    check_relative_invariance(oracle.rope3d_ref)


def test_rope_depends_on_differences_not_absolute():
    # Scores for two tokens with equal coordinate differences but different frames: identical;
    # a change of difference changes the score (the rotation is not trivial).
    grid = (4, 4, 4)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 1, 128))
    x[:] = x[0]
    y = oracle.rope3d_ref(x, grid, 0, (44, 42, 42))
    n_of = lambda t, h, w: (t * 4 + h) * 4 + w
    s1 = y[n_of(0, 1, 2), 0] @ y[n_of(1, 2, 3), 0]
    s2 = y[n_of(2, 0, 0), 0] @ y[n_of(3, 1, 1), 0]
    s3 = y[n_of(2, 0, 0), 0] @ y[n_of(3, 1, 2), 0]
    assert s1 == pytest.approx(s2, abs=1e-11)
    assert abs(s1 - s3) > 1e-3


def test_rope_identity_at_origin_and_text_rows():
    x = np.random.default_rng(7).standard_normal((72 + 5, 2, 128))
    y = oracle.rope3d_ref(x, (3, 4, 6), 5, (44, 42, 42))
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_array_equal(y[72:], x[72:])
    assert np.abs(y[1] - x[1]).max() > 1e-3


def test_rope_t_range_only_moves_with_t():
    # Channels of the t range change only with t; the h and w ranges never move with t.
    grid, split = (5, 3, 4), (44, 42, 42)
    x = np.random.default_rng(8).standard_normal((60, 1, 128))
    x[:] = x[0]
    y = oracle.rope3d_ref(x, grid, 0, split)
    same_hw = [(t * 3 + 1) * 4 + 2 for t in range(5)]
    for n in same_hw[1:]:
        np.testing.assert_allclose(y[n, 0, 44:], y[same_hw[0], 0, 44:], atol=1e-14)
        assert np.abs(y[n, 0, :44] - y[same_hw[0], 0, :44]).max() > 1e-3


# The frequency ladder.  No page prints a frequency: the first page calls the scheme "FLUX's 2D
# RoPE plus a time dimension" ("A video model's architecture: spatiotemporal attention and the 3D
# VAE", "Position: RoPE in three dimensions"), i.e. one independent 1D RoPE per axis range.  An
# independent implementation of exactly that is importable here: the per-axis rotary embedding of
# V-JEPA 2 in `transformers`, which rotates each axis range of D channels with its own ladder
# over D.  Its channel pairing and frequency placement differ from the oracle's, so only the
# ladder is compared, read back from the routine's output on unit vectors at position 1.

def _vjepa2_axis_ladder(D):
    """omega_k, k < D/2, of V-JEPA 2's rotary embedding of a D-channel axis range (theta 1e4).

    Row k < D/2 of the routine's matrix at position 1 carries frequency index k on its diagonal
    (cos) and in its pair partner's column (sin, signed by the pair side); the angle is then
    atan2(sin, cos), unambiguous since every omega <= 1 < pi.
    """
    from transformers.models.vjepa2.modeling_vjepa2 import rotate_queries_or_keys
    x = torch.eye(D, dtype=torch.float64).reshape(1, 1, D, D)     # token c holds unit vector e_c
    pos = torch.ones(1, 1, D, dtype=torch.float64)
    m = rotate_queries_or_keys(x, pos)[0, 0].T.numpy()             # m[r, c]: channel r of R e_c
    om = np.empty(D // 2)
    for kk in range(D // 2):
        s = m[kk, kk - 1] if kk % 2 else -m[kk, kk + 1]
        om[kk] = math.atan2(s, m[kk, kk])
    return om


LADDER_SPLITS = [(44, 42, 42), (16, 56, 56)]


def check_ladder(freq_fn):
    for split in LADDER_SPLITS:
        freqs = freq_fn(split, 10000.0)
        for axis, da in enumerate(split):
            np.testing.assert_allclose(freqs[axis], _vjepa2_axis_ladder(da), rtol=1e-12, atol=0)


def check_rope_turns_by_ladder(rope_fn):
    # The rotation itself: a unit vector on the first channel of pair j of axis a, at the row whose
    # coordinate on a is 1 and 0 on the other two, must turn by exactly the independent omega_{a,j}.
    grid = (2, 2, 2)
    for split in LADDER_SPLITS:
        off = 0
        for axis, da in enumerate(split):
            row = (4, 2, 1)[axis]                       # (1,0,0), (0,1,0), (0,0,1) in flat order
            ladder = _vjepa2_axis_ladder(da)
            x = np.zeros((8, da // 2, 128))
            for j in range(da // 2):
                x[row, j, off + 2 * j] = 1.0
            y = rope_fn(x, grid, 0, split, 10000.0)
            for j in range(da // 2):
                ang = math.atan2(y[row, j, off + 2 * j + 1], y[row, j, off + 2 * j])
                assert ang == pytest.approx(ladder[j], rel=1e-12, abs=1e-15)
            off += da


def test_rope_frequency_ladder_matches_independent_axis_rope():
    check_ladder(oracle.rope_frequencies)


def test_rope_rotation_uses_the_independent_ladder():
    check_rope_turns_by_ladder(oracle.rope3d_ref)


def test_rope_ladder_probe_reads_known_endpoints():
    # The probe itself, on closed forms: omega_0 = 1 for every range, and for D = 16 the ladder
    # is 10^(-k/2) exactly (10000^(-2k/16)).
    for D in (16, 42, 44, 56):
        assert _vjepa2_axis_ladder(D)[0] == pytest.approx(1.0, abs=1e-15)
    np.testing.assert_allclose(_vjepa2_axis_ladder(16), 10.0 ** (-np.arange(8) / 2.0), rtol=1e-12)


# ------------------------------------------------------------------------------------------
# Attention
# ------------------------------------------------------------------------------------------

def _sdpa(qr, kr, v, mask=None):
    q = torch.from_numpy(np.ascontiguousarray(qr.transpose(1, 0, 2)))
    k = torch.from_numpy(np.ascontiguousarray(kr.transpose(1, 0, 2)))
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=m)
    return o.numpy().transpose(1, 0, 2)


def check_full_vs_sdpa(full_fn):
    grid, n_text = (3, 4, 6), 5
    x = make_qkv(77, 2, 128, 11, "f32")
    out = full_fn(x.q, x.k, x.v, grid, n_text, (44, 42, 42), 10000.0)
    qr = oracle.rope3d_ref(x.q.astype(np.float64), grid, n_text)
    kr = oracle.rope3d_ref(x.k.astype(np.float64), grid, n_text)
    ref = _sdpa(qr, kr, x.v.astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_full_attention_matches_torch_sdpa():
    check_full_vs_sdpa(oracle.full_attention_ref)


def test_full_attention_no_rope_ranges_reduce_to_plain_sdpa():
    # Grid 1x1x1 plus text rows: the only video row sits at the origin (identity), text rows are
    # not rotated, so the whole computation is plain attention on the raw inputs.
    x = make_qkv(1 + 9, 3, 128, 12, "f32")
    out = oracle.full_attention_ref(x.q, x.k, x.v, (1, 1, 1), 9)
    ref = _sdpa(x.q.astype(np.float64), x.k.astype(np.float64), x.v.astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_rows_subset_equals_dense():
    grid = (3, 5, 7)
    x = make_qkv(105, 2, 128, 13, "f32")
    dense = oracle.full_attention_ref(x.q, x.k, x.v, grid)
    rows = np.array([0, 1, 34, 35, 70, 104])
    sub = oracle.full_attention_ref(x.q, x.k, x.v, grid, rows=rows)
    np.testing.assert_allclose(sub, dense[rows], rtol=0, atol=1e-13)
    sub2 = oracle.full_attention_ref(x.q, x.k, x.v, grid, rows=rows, heads=[1])
    np.testing.assert_allclose(sub2[:, 0], dense[rows, 1], rtol=0, atol=1e-13)


def test_constant_values_give_constant_output():
    x = make_qkv(72, 2, 128, 14, "f32")
    v = np.full_like(x.v, 0.0) + np.arange(128, dtype=np.float32)[None, None, :]
    out = oracle.full_attention_ref(x.q, x.k, v, (3, 4, 6))
    np.testing.assert_allclose(out, np.broadcast_to(v[:1], out.shape), rtol=1e-13, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    x = make_qkv(72, 2, 128, 15, "f32")
    q = np.zeros_like(x.q)
    out = oracle.full_attention_ref(q, x.k, x.v, (3, 4, 6))
    mean = x.v.astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-13)


def test_peaked_query_selects_one_value():
    grid = (2, 3, 4)
    x = make_qkv(24, 1, 128, 16, "f32")
    kr = oracle.rope3d_ref(x.k.astype(np.float64), grid)
    j = 17
    # Query row 5 chosen so that its rotated vector is alpha * k~_j: rotate back with R(p_5)^T.
    t, h, w, _ = oracle.token_positions(grid)
    r5 = _r3d_matrix((t[5], h[5], w[5]), (44, 42, 42), 10000.0)
    q = x.q.astype(np.float64).copy()
    q[5, 0] = r5.T @ (40.0 * kr[j, 0])
    out = oracle.full_attention_ref(q, x.k, x.v, grid, rows=[5])
    np.testing.assert_allclose(out[0, 0], x.v[j, 0], atol=1e-6)


def test_softmax_weights_sum_to_one():
    # With v = ones in one channel and zeros elsewhere the output is the row sum of P.
    x = make_qkv(105, 2, 128, 17, "f32")
    v = np.zeros_like(x.v)
    v[:, :, 3] = 1.0
    out = oracle.full_attention_ref(x.q * 6, x.k, v, (3, 5, 7))
    np.testing.assert_allclose(out[:, :, 3], 1.0, rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------------
# Factorised
# ------------------------------------------------------------------------------------------

def check_factorized_vs_masked_sdpa(fact_fn):
    grid = (3, 4, 6)
    x = make_qkv(72, 2, 128, 18, "f32")
    out = fact_fn(x.q, x.k, x.v, grid, (44, 42, 42), 10000.0)
    t, h, w, _ = oracle.token_positions(grid)
    qr = oracle.rope3d_ref(x.q.astype(np.float64), grid)
    kr = oracle.rope3d_ref(x.k.astype(np.float64), grid)
    same_t = t[:, None] == t[None, :]
    same_hw = (h[:, None] == h[None, :]) & (w[:, None] == w[None, :])
    o_s = _sdpa(qr, kr, x.v.astype(np.float64), same_t)
    ref = _sdpa(qr, kr, o_s, same_hw)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_factorized_equals_masked_full_composition():
    check_factorized_vs_masked_sdpa(oracle.factorized_ref)


def test_factorized_equals_full_when_one_frame():
    grid = (1, 5, 7)
    x = make_qkv(35, 2, 128, 19, "f32")
    np.testing.assert_allclose(oracle.factorized_ref(x.q, x.k, x.v, grid),
                               oracle.full_attention_ref(x.q, x.k, x.v, grid), rtol=0, atol=1e-13)


def test_factorized_equals_full_when_one_position():
    grid = (9, 1, 1)
    x = make_qkv(9, 2, 128, 20, "f32")
    np.testing.assert_allclose(oracle.factorized_ref(x.q, x.k, x.v, grid),
                               oracle.full_attention_ref(x.q, x.k, x.v, grid), rtol=0, atol=1e-13)


def test_factorized_rows_subset():
    grid = (4, 3, 5)
    x = make_qkv(60, 2, 128, 21, "f32")
    dense = oracle.factorized_ref(x.q, x.k, x.v, grid)
    rows = np.array([0, 7, 14, 15, 44, 59])
    np.testing.assert_allclose(oracle.factorized_ref(x.q, x.k, x.v, grid, rows=rows), dense[rows],
                               rtol=0, atol=1e-13)


def test_factorized_spatial_stage_ignores_t_range():
    # Inside one frame R_t(t)^T R_t(t) = I: the spatial stage is the same with the t range unrotated.
    grid = (3, 4, 5)
    x = make_qkv(60, 1, 128, 22, "f32")
    _, o_s = oracle.factorized_ref(x.q, x.k, x.v, grid, return_spatial=True)
    split_hw = (44, 42, 42)
    t, h, w, _ = oracle.token_positions(grid)
    qr = oracle.rope3d_ref(x.q.astype(np.float64), grid, 0, split_hw)
    kr = oracle.rope3d_ref(x.k.astype(np.float64), grid, 0, split_hw)
    # undo the t rotation on both sides (positions reset to t = 0 -> identity on channels < 44)
    qr[:, :, :44] = x.q[:, :, :44]
    kr[:, :, :44] = x.k[:, :, :44]
    for tt in range(3):
        rows = np.arange(tt * 20, (tt + 1) * 20)
        ref = oracle.attention_dense(qr[rows], kr[rows], x.v[rows].astype(np.float64))
        got = np.stack([o_s[int(r)] for r in rows])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin above
# ------------------------------------------------------------------------------------------

def _fails(check, fn):
    try:
        check(fn)
    except AssertionError:
        return True
    return False


def _mut_positions_w_slowest(grid, n_text=0):
    t_, h_, w_ = grid
    n = np.arange(t_ * h_ * w_)
    t, h, w, vid = so.token_positions(grid, n_text)
    t[:n.size], h[:n.size], w[:n.size] = n % t_, (n // t_) % h_, n // (t_ * h_)
    return t, h, w, vid


def _rope_variant(mode):
    def fn(x, grid, n_text=0, split=(44, 42, 42), theta=10000.0, rows=None):
        t, h, w, vid = so.token_positions(grid, n_text)
        freqs = so.rope_frequencies(split, theta)
        y = np.array(x, dtype=np.float64, copy=True)
        off = 0
        for axis, da in enumerate(split):
            pos = (t, h, w)[axis]
            for j in range(da // 2):
                if mode == "half_split":
                    c0, c1 = off + j, off + j + da // 2
                else:
                    c0, c1 = off + 2 * j, off + 2 * j + 1
                phi = pos * freqs[axis][j]
                if mode == "axis_swap":
                    phi = (t, w, h)[axis] * freqs[axis][j]
                c, s = np.cos(phi)[:, None], np.sin(phi)[:, None]
                if mode == "sign":
                    s = -s
                x0, x1 = x[:, :, c0], x[:, :, c1]
                y[:, :, c0] = x0 * c - x1 * s
                y[:, :, c1] = x0 * s + x1 * c
                if mode == "dropped_term":
                    y[:, :, c1] = x1 * c
            off += da
        return y
    return fn


def _full_variant(mode):
    def fn(q, k, v, grid, n_text=0, split=(44, 42, 42), theta=10000.0):
        qr = so.rope3d_ref(np.asarray(q, np.float64), grid, n_text, split, theta)
        kr = so.rope3d_ref(np.asarray(k, np.float64), grid, n_text, split, theta)
        if mode == "no_scale":
            qr = qr * math.sqrt(128)
        if mode == "rope_on_v":
            v = so.rope3d_ref(np.asarray(v, np.float64), grid, n_text, split, theta)
        if mode == "transposed":
            return so.attention_dense(kr, qr, np.asarray(v, np.float64))
        return so.attention_dense(qr, kr, np.asarray(v, np.float64))
    return fn


def _fact_variant(mode):
    def fn(q, k, v, grid, split=(44, 42, 42), theta=10000.0):
        t, h, w, _ = so.token_positions(grid)
        qr = so.rope3d_ref(np.asarray(q, np.float64), grid, 0, split, theta)
        kr = so.rope3d_ref(np.asarray(k, np.float64), grid, 0, split, theta)
        same_t = t[:, None] == t[None, :]
        same_hw = (h[:, None] == h[None, :]) & (w[:, None] == w[None, :])
        vv = np.asarray(v, np.float64)
        if mode == "temporal_first":
            return so.attention_dense(qr, kr, so.attention_dense(qr, kr, vv, same_hw), same_t)
        if mode == "stage2_raw_values":
            return so.attention_dense(qr, kr, vv, same_hw)
        raise ValueError(mode)
    return fn


@pytest.mark.parametrize("mode", ["half_split", "sign", "axis_swap", "dropped_term"])
def test_planted_rope_mistakes_are_caught(mode):
    fn = _rope_variant(mode)
    caught = _fails(check_rope_against_matrix, fn)
    if mode == "dropped_term":
        caught = caught or _fails(check_relative_invariance, fn)
    assert caught, f"rope mutant {mode} passed the pins"
    # the unmutated form of the same helper passes
    assert not _fails(check_rope_against_matrix, _rope_variant("none"))


def test_planted_flat_order_mistake_is_caught():
    assert _fails(check_shards, _mut_positions_w_slowest)


def _ladder_variant(mode):
    """Frequency ladders with a planted mistake: the exponent without its factor 2, one exponent
    over the whole head (pair index counted from the head's first pair), j counted from 1."""
    def fn(split, theta=10000.0):
        d = sum(split)
        out, first = [], 0
        for da in split:
            j = np.arange(da // 2, dtype=np.float64)
            if mode == "no_factor_2":
                om = theta ** (-j / da)
            elif mode == "global_exponent":
                om = theta ** (-2.0 * (first + j) / d)
            elif mode == "j_from_1":
                om = theta ** (-2.0 * (j + 1) / da)
            else:
                om = theta ** (-2.0 * j / da)
            out.append(om)
            first += da // 2
        return out
    return fn


def _rope_with_ladder(freq_fn):
    """The oracle's rotation with its frequency ladder replaced."""
    def fn(x, grid, n_text=0, split=(44, 42, 42), theta=10000.0, rows=None):
        t, h, w, vid = so.token_positions(grid, n_text)
        freqs = freq_fn(split, theta)
        y = np.array(x, dtype=np.float64, copy=True)
        for axis, j, c0 in so.rope_pair_layout(split):
            phi = (t, h, w)[axis] * freqs[axis][j]
            c = np.where(vid, np.cos(phi), 1.0)[:, None]
            s = np.where(vid, np.sin(phi), 0.0)[:, None]
            x0, x1 = x[:, :, c0], x[:, :, c0 + 1]
            y[:, :, c0] = x0 * c - x1 * s
            y[:, :, c0 + 1] = x0 * s + x1 * c
        return y
    return fn


@pytest.mark.parametrize("mode", ["no_factor_2", "global_exponent", "j_from_1"])
def test_planted_ladder_mistakes_are_caught(mode):
    assert _fails(check_ladder, _ladder_variant(mode)), f"ladder mutant {mode} passed the pin"
    assert _fails(check_rope_turns_by_ladder, _rope_with_ladder(_ladder_variant(mode)))
    # the unmutated forms of the same helpers pass
    assert not _fails(check_ladder, _ladder_variant("none"))
    assert not _fails(check_rope_turns_by_ladder, _rope_with_ladder(_ladder_variant("none")))


@pytest.mark.parametrize("mode", ["no_scale", "rope_on_v", "transposed"])
def test_planted_attention_mistakes_are_caught(mode):
    assert _fails(check_full_vs_sdpa, _full_variant(mode))
    assert not _fails(check_full_vs_sdpa, _full_variant("none"))


@pytest.mark.parametrize("mode", ["temporal_first", "stage2_raw_values"])
def test_planted_factorized_mistakes_are_caught(mode):
    assert _fails(check_factorized_vs_masked_sdpa, _fact_variant(mode))


def test_planted_cost_model_mistake_is_caught():
    def no_temporal_term(grid, hidden, layers=1):
        r = dict(oracle.attn_flop_model(grid, hidden, layers))
        t, s = grid[0], grid[1] * grid[2]
        r["factorized"] -= layers * s * 4 * t * t * hidden
        return r
    assert _fails(check_flop_table, no_temporal_term)


# ---- text cross-attention, partial attention and merge -----------------------------------------

def _sdpa64(q, k, v):
    """torch SDPA in float64 on [N, heads, d] arrays (heads as the batch)."""
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(q, (1, 0, 2))))
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(k, (1, 0, 2))))
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(v, (1, 0, 2))))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return np.transpose(o.numpy(), (1, 0, 2))


def test_cross_attention_matches_torch_sdpa_rectangular():
    rng = np.random.default_rng(71)
    q = rng.standard_normal((37, 3, 16))
    k = rng.standard_normal((11, 3, 16))
    v = rng.standard_normal((11, 3, 16))
    got = oracle.cross_attention_ref(q, k, v)
    np.testing.assert_allclose(got, _sdpa64(q, k, v), rtol=1e-12, atol=1e-12)
    rows = np.array([0, 5, 36])
    np.testing.assert_allclose(oracle.cross_attention_ref(q, k, v, rows=rows), got[rows], rtol=0, atol=0)


def test_cross_attention_single_key_returns_its_value_and_ignores_key_order():
    rng = np.random.default_rng(72)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    np.testing.assert_allclose(oracle.cross_attention_ref(q, k, v), np.broadcast_to(v, (5, 2, 8)), atol=1e-15)
    k2 = rng.standard_normal((9, 2, 8))
    v2 = rng.standard_normal((9, 2, 8))
    perm = rng.permutation(9)
    np.testing.assert_allclose(oracle.cross_attention_ref(q, k2, v2),
                               oracle.cross_attention_ref(q, k2[perm], v2[perm]), rtol=1e-13, atol=1e-14)


def _grid_inputs(seed, grid, n_text, heads, d):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2] + n_text
    return (rng.standard_normal((n, heads, d)), rng.standard_normal((n, heads, d)),
            rng.standard_normal((n, heads, d)))


def test_partial_over_all_keys_matches_sdpa_and_logsumexp():
    grid, n_text, heads, d, split = (2, 3, 4), 3, 2, 16, (4, 6, 6)
    q, k, v = _grid_inputs(73, grid, n_text, heads, d)
    o, lse = oracle.partial_attention_ref(q, k, v, grid, n_text, split)
    qr = oracle.rope3d_ref(q, grid, n_text, split)
    kr = oracle.rope3d_ref(k, grid, n_text, split)
    np.testing.assert_allclose(o, _sdpa64(qr, kr, v), rtol=1e-12, atol=1e-12)
    s = torch.einsum("nhd,mhd->hnm", torch.from_numpy(qr), torch.from_numpy(kr)) / math.sqrt(d)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy().T, rtol=1e-12, atol=1e-12)


def test_merge_of_key_runs_equals_sdpa_over_all_keys():
    grid, n_text, heads, d, split = (3, 2, 3), 2, 2, 16, (4, 6, 6)
    q, k, v = _grid_inputs(74, grid, n_text, heads, d)
    n = q.shape[0]
    qb, qc = 4, 9                       # a run of queries with its global offset
    cuts = [0, 5, 6, 13, n]             # uneven runs of keys, one of a single row
    parts = [oracle.partial_attention_ref(q[qb:qb + qc], k[a:b], v[a:b], grid, n_text, split,
                                          q_begin=qb, kv_begin=a) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle.merge_partials_ref(parts)
    qr = oracle.rope3d_ref(q, grid, n_text, split)[qb:qb + qc]
    kr = oracle.rope3d_ref(k, grid, n_text, split)
    np.testing.assert_allclose(o, _sdpa64(qr, kr, v), rtol=1e-12, atol=1e-12)
    s = torch.einsum("nhd,mhd->hnm", torch.from_numpy(qr), torch.from_numpy(kr)) / math.sqrt(d)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy().T, rtol=1e-12, atol=1e-12)
    # order of the parts does not matter; one part merges to itself
    o2, lse2 = oracle.merge_partials_ref(parts[::-1])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)
    o1, l1 = oracle.merge_partials_ref(parts[:1])
    np.testing.assert_allclose(o1, parts[0][0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l1, parts[0][1], rtol=0, atol=1e-15)


def test_partial_uses_global_positions():
    """The same key rows give different results when their global offset changes (RoPE)."""
    grid, heads, d, split = (4, 2, 2), 1, 8, (4, 2, 2)
    q, k, v = _grid_inputs(75, grid, 0, heads, d)
    a = oracle.partial_attention_ref(q[:4], k[4:8], v[4:8], grid, 0, split, q_begin=0, kv_begin=4)
    b = oracle.partial_attention_ref(q[:4], k[4:8], v[4:8], grid, 0, split, q_begin=0, kv_begin=8)
    assert np.abs(a[1] - b[1]).max() > 1e-3


@pytest.mark.parametrize("mode", ["no_shift", "lse_base2", "unweighted"])
def test_planted_merge_mistakes_are_caught(mode):
    grid, n_text, heads, d, split = (2, 2, 3), 0, 2, 8, (4, 2, 2)
    q, k, v = _grid_inputs(76, grid, n_text, heads, d)
    parts = [oracle.partial_attention_ref(q, k[a:b], v[a:b], grid, n_text, split, kv_begin=a)
             for a, b in [(0, 5), (5, 12)]]
    lses = np.stack([l for _, l in parts])
    if mode == "no_shift":
        w = np.exp(lses)
        o = sum(w[i][:, :, None] * parts[i][0] for i in range(2))
    elif mode == "lse_base2":
        w = 2.0 ** lses
        o = sum((w[i] / w.sum(0))[:, :, None] * parts[i][0] for i in range(2))
    else:
        o = 0.5 * (parts[0][0] + parts[1][0])
    qr = oracle.rope3d_ref(q, grid, n_text, split)
    kr = oracle.rope3d_ref(k, grid, n_text, split)
    assert np.abs(o - _sdpa64(qr, kr, v)).max() > 1e-3


# ---- QKV projection with the rotation of its output ---------------------------------------------

def test_qkv_projection_matches_explicit_sums():
    """The product part against plain nested sums (no matrix routine); with T' = 1 and the whole
    head in the t range every row sits at t = 0, so nothing is rotated."""
    rng = np.random.default_rng(81)
    grid, heads, d = (1, 2, 2), 2, 4
    n, c = 4, heads * d
    x = rng.standard_normal((n, c))
    w = rng.standard_normal((3 * c, c))
    b = rng.standard_normal(3 * c)
    q, k, v = oracle.qkv_rope_ref(x, w, b, grid, 0, (4, 0, 0))
    for r in range(n):
        for f in range(3 * c):
            acc = b[f]
            for i in range(c):
                acc += x[r, i] * w[f, i]
            sec, rem = divmod(f, c)
            got = (q, k, v)[sec][r, rem // d, rem % d]
            assert abs(got - acc) < 1e-12


def test_qkv_rope_rotates_q_and_k_only_and_bias_passes_through():
    rng = np.random.default_rng(82)
    grid, split, heads = (2, 2, 3), (4, 2, 2), 2
    c = heads * 8
    n = 12
    x = rng.standard_normal((n, c))
    w = np.zeros((3 * c, c))
    b = rng.standard_normal(3 * c)
    q, k, v = oracle.qkv_rope_ref(x, w, b, grid, 0, split)
    bq = np.broadcast_to(b[:c].reshape(1, heads, 8), (n, heads, 8))
    np.testing.assert_allclose(q, oracle.rope3d_ref(bq, grid, 0, split), atol=1e-14)
    np.testing.assert_allclose(v, np.broadcast_to(b[2 * c:].reshape(1, heads, 8), (n, heads, 8)), atol=0)
    # row 0 sits at the origin: no rotation there
    np.testing.assert_allclose(k[0], b[c:2 * c].reshape(heads, 8), atol=1e-15)


def test_qkv_rope_then_plain_attention_equals_full_attention():
    """Projection + rotation, then attention without rotation == full 3D-RoPE attention of x W."""
    rng = np.random.default_rng(83)
    grid, n_text, split, heads, d = (2, 3, 2), 3, (4, 2, 2), 2, 8
    c = heads * d
    n = grid[0] * grid[1] * grid[2] + n_text
    x = rng.standard_normal((n, c))
    w = rng.standard_normal((3 * c, c)) / np.sqrt(c)
    q, k, v = oracle.qkv_rope_ref(x, w, None, grid, n_text, split)
    got = oracle.cross_attention_ref(q, k, v)
    y = x @ w.T
    ref = oracle.full_attention_ref(y[:, :c].reshape(n, heads, d), y[:, c:2 * c].reshape(n, heads, d),
                                    y[:, 2 * c:].reshape(n, heads, d), grid, n_text, split)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([1, 7, n - 1])
    qs, ks, vs = oracle.qkv_rope_ref(x, w, None, grid, n_text, split, rows=rows)
    np.testing.assert_allclose(qs, q[rows], atol=0)
    np.testing.assert_allclose(vs, v[rows], atol=0)


@pytest.mark.parametrize("mode", ["w_not_transposed", "sections_swapped"])
def test_planted_qkv_mistakes_are_caught(mode):
    rng = np.random.default_rng(84)
    grid, split, heads, d = (1, 2, 2), (4, 0, 0), 1, 4
    c = heads * d
    x = rng.standard_normal((4, c))
    w = rng.standard_normal((3 * c, c))
    q, k, v = oracle.qkv_rope_ref(x, w, None, grid, 0, split)
    if mode == "w_not_transposed":
        y = x @ w[:c]
        assert np.abs(y.reshape(4, heads, d) - q).max() > 1e-3
    else:
        y = x @ w[c:2 * c].T
        assert np.abs(y.reshape(4, heads, d) - q).max() > 1e-3


# ---- local 3D-window attention ---------------------------------------------------------------------

def test_window_attention_equals_masked_sdpa():
    """Against torch SDPA with an explicit same-window boolean mask (an independent routine)."""
    rng = np.random.default_rng(91)
    grid, window, split, heads, d = (4, 4, 6), (2, 2, 3), (4, 2, 2), 2, 8
    n = 96
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    got = oracle.window_attention_ref(q, k, v, grid, window, split)
    t, h, w, _ = oracle.token_positions(grid)
    key = np.stack([t // 2, h // 2, w // 3], 1)
    mask = (key[:, None, :] == key[None, :, :]).all(-1)
    qr = oracle.rope3d_ref(q, grid, 0, split)
    kr = oracle.rope3d_ref(k, grid, 0, split)
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(qr, (1, 0, 2))))
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(kr, (1, 0, 2))))
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(v, (1, 0, 2))))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    np.testing.assert_allclose(got, np.transpose(ref.numpy(), (1, 0, 2)), rtol=1e-12, atol=1e-12)
    rows = np.array([0, 17, 95])
    np.testing.assert_allclose(oracle.window_attention_ref(q, k, v, grid, window, split, rows=rows), got[rows], atol=0)


def test_window_attention_special_cases():
    rng = np.random.default_rng(92)
    grid, split, heads, d = (3, 4, 4), (4, 2, 2), 2, 8
    n = 48
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    # one window over the whole grid is full attention
    np.testing.assert_allclose(oracle.window_attention_ref(q, k, v, grid, grid, split),
                               oracle.full_attention_ref(q, k, v, grid, 0, split), rtol=1e-12, atol=1e-12)
    # (1, H', W') windows are the factorised spatial stage
    _, o_s = oracle.factorized_ref(q, k, v, grid, split, return_spatial=True)
    spatial = np.stack([o_s[i] for i in range(n)])
    np.testing.assert_allclose(oracle.window_attention_ref(q, k, v, grid, (1, 4, 4), split), spatial,
                               rtol=1e-12, atol=1e-12)
    # 1 x 1 x 1 windows: every token sees only itself
    np.testing.assert_allclose(oracle.window_attention_ref(q, k, v, grid, (1, 1, 1), split), v, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.window_attention_ref(q, k, v, grid, (2, 4, 4), split)
