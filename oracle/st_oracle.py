"""Plain float64 CPU oracle: 3D RoPE, full spatiotemporal softmax attention, factorised attention.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's CPU-baseline leg,
never by the library.  It shares no code, header, table or constant with the HIP path.

What it computes, and where each step comes from (page title, then section):

* Token grid -- "A video model's architecture: spatiotemporal attention and the 3D VAE",
  self-test answer 1 and section "The latents: the extra time axis": the first frame is its own
  latent frame and every 4 frames after it make one more; space shrinks 8x per side; tokens are
  1x2x2 patches of that latent grid.
* Flat token order -- same page, section "Position: RoPE in three dimensions": token coordinates
  are enumerated with t slowest and w fastest (the printed per-card shards list (0,0,0), (0,0,1),
  (0,0,2), (0,1,0), ...), so flat index n = (t*H' + h)*W' + w.
* 3D RoPE -- same page, self-test answer 4 and "Position: RoPE in three dimensions" (the head
  dimension is split into three ranges rotated by t, h and w); "CogVideoX Architecture: 3D Causal
  VAE Compression, ...", section "3. 3D Rotary Position Embeddings (3D RoPE)" (the rotation is the
  block-diagonal diag(R_t(t), R_y(y), R_x(x)) and scores depend only on coordinate differences);
  "How AI Generates Video: Inside Sora and Wan2.1 on a Real GPU", FAQ "What is 3D RoPE in video
  diffusion transformers?" (Wan's 128-dim head uses 22/21/21 rotation pairs, axes_dim 44/42/42).
* Full attention -- the first page, self-test answer 2 and "How attention sees time: factorised or
  full": every token attends to every token together; non-causal softmax(q k^T / sqrt(d)) v.
* Factorised attention -- same passage: spatial attention inside each frame (T' sequences of
  length H'W'), then temporal attention at each spatial position (H'W' sequences of length T').
* Cost model -- same section's per-layer formulas (full 4 (T' n_sp)^2 D, factorised
  T' 4 n_sp^2 D + n_sp 4 T'^2 D, linear 24 N D^2).
* Text cross-attention -- "04 · HunyuanVideo 与 Wan", section 3.1 (one Wan block step by step):
  queries come from the video tokens, keys and values from the text condition (at most 512
  tokens, same section), and the text is not updated by this step.
* QKV projection with the 3D rotation applied to its output -- "04 · HunyuanVideo 与 Wan", section
  3.1 (the Wan block's projections Q = X W_Q, K = X W_K, V = X W_V) and the first page's cost
  model (the linear layers, 24 N D^2 per layer, of which the QKV projection is 6 N D^2); the
  rotation is the same 3D RoPE of q and k, applied to the projection's output.
* Local 3D-window attention -- the CogVideoX record page (the W.A.L.T comparison alternates
  per-frame spatial blocks with local 3D-window blocks): the grid is cut into non-overlapping
  windows of wt x wh x ww tokens and every token attends to the tokens of its own window, with
  the same rotated q and k.  Full attention is the one-window case and the factorised spatial
  stage the (1, H', W') case.
* Partial attention and its merge -- the CogVideoX record page ("Budget for that cost, because it
  grows": attention is split across devices by context parallelism, 2D ring and Ulysses) and the
  first page's shard listing under "Position: RoPE in three dimensions" (each device holds a
  contiguous run of tokens whose (t, h, w) are absolute).  A device that sees only a run of keys
  returns its normalised output and the log of its softmax denominator; the exact result over
  all keys is their log-sum-exp weighted combination (the standard online-softmax identity).

Readings where the pages are silent (each one is also listed in the design notes):

* RoPE pairs are interleaved, channels (off + 2j, off + 2j + 1) inside each contiguous range, ranges
  in the order t, h, w; pair j of an axis with range size d_a turns by pos * theta^(-2j / d_a)
  (each axis an independent 1D RoPE, theta = 10000); the turn is counter-clockwise:
  (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).  The frequency ladder is pinned against an
  independent per-axis rotary embedding (V-JEPA 2's, in `transformers`), both as a list and as the
  angle each pair of the rotation turns by.  The pairing and the sign remain readings beyond the
  structural pins (block-diagonal form, norm preservation, relative-position invariance, identity
  at the origin): no page prints a rotated vector.
* Text tokens, when present, come after all video tokens and are not rotated.
* The factorised second stage uses the same rotated q and k and takes the first stage's output as
  its values.
* Absolute attention outputs on random inputs: no page prints one, so the tests pin them by
  special cases, invariants and an independent library routine (torch's scaled_dot_product_attention
  in float64).
* Cross-attention applies no rotation: the page gives 3D RoPE for the video self-attention and none
  for the text keys.  The log-sum-exp of a partial result is natural-log, over scaled scores
  s / sqrt(d).
"""
from __future__ import annotations

import math

import numpy as np

ORACLE_DTYPE = np.float64

__all__ = [
    "ORACLE_DTYPE",
    "latent_token_grid",
    "attn_flop_model",
    "metric_flops",
    "factorized_flops",
    "token_positions",
    "rope_pair_layout",
    "rope_frequencies",
    "rope3d_ref",
    "attention_dense",
    "attention_rows",
    "full_attention_ref",
    "factorized_ref",
    "cross_attention_ref",
    "partial_attention_ref",
    "merge_partials_ref",
    "qkv_rope_ref",
    "window_attention_ref",
]


# --------------------------------------------------------------------------------------------
# Shapes and cost model
# --------------------------------------------------------------------------------------------

def latent_token_grid(frames: int, height: int, width: int, t_ratio: int = 4, s_ratio: int = 8,
                      patch_t: int = 1, patch_s: int = 2, latent_channels: int = 16):
    """Video size -> (latent T, H, W), token grid (T', H', W'), token count, token dimension.

    From the first page's self-test answer 1 and "The latents: the extra time axis": the time
    axis keeps the first frame alone and folds every ``t_ratio`` later frames into one latent
    frame; each spatial side shrinks by ``s_ratio``; the denoiser then cuts 1x2x2 patches, so a
    token carries latent_channels * 1 * 2 * 2 values.
    """
    t_lat = 1 + (frames - 1) // t_ratio
    h_lat = height // s_ratio
    w_lat = width // s_ratio
    grid = (t_lat // patch_t, h_lat // patch_s, w_lat // patch_s)
    n = grid[0] * grid[1] * grid[2]
    return (t_lat, h_lat, w_lat), grid, n, latent_channels * patch_t * patch_s * patch_s


def attn_flop_model(grid, hidden: int, layers: int = 1):
    """Per-step FLOP of full and factorised attention and of the linear layers.

    First page, "How attention sees time: factorised or full": with S = H'W' tokens per frame and
    D the hidden width, full attention costs 4 (T' S)^2 D per layer, factorised costs
    T' * 4 S^2 D + S * 4 T'^2 D, and the linear layers cost 24 N D^2 per layer.
    """
    t, h, w = grid
    s = h * w
    n = t * s
    full = 4 * (t * s) ** 2 * hidden
    fact = t * 4 * s ** 2 * hidden + s * 4 * t ** 2 * hidden
    linear = 24 * n * hidden ** 2
    return {"full": layers * full, "factorized": layers * fact, "linear": layers * linear}


def metric_flops(n_tokens: int, heads: int, d: int) -> int:
    """FLOP counted for one full-attention forward: 4 N^2 heads d (q k^T plus P v, no softmax)."""
    return 4 * n_tokens * n_tokens * heads * d


def factorized_flops(grid, heads: int, d: int) -> int:
    """FLOP counted for one factorised forward (spatial plus temporal), same counting rule."""
    t, h, w = grid
    s = h * w
    return 4 * t * s * s * heads * d + 4 * s * t * t * heads * d


# --------------------------------------------------------------------------------------------
# Positions and RoPE
# --------------------------------------------------------------------------------------------

def token_positions(grid, n_text: int = 0):
    """(t, h, w) of every row and a mask of video rows, for N = T'H'W' + n_text rows.

    Flat order n = (t*H' + h)*W' + w (first page, "Position: RoPE in three dimensions": the
    coordinate list runs over t, then h, then w, as the printed shards show).  Text rows follow the
    video rows and carry no position (their mask entry is False; their coordinates are 0).
    """
    t_, h_, w_ = grid
    nv = t_ * h_ * w_
    n = nv + n_text
    t = np.zeros(n, dtype=np.int64)
    h = np.zeros(n, dtype=np.int64)
    w = np.zeros(n, dtype=np.int64)
    k = 0
    for ti in range(t_):
        for hi in range(h_):
            for wi in range(w_):
                t[k], h[k], w[k] = ti, hi, wi
                k += 1
    is_video = np.zeros(n, dtype=bool)
    is_video[:nv] = True
    return t, h, w, is_video


def rope_pair_layout(split):
    """Pairs of channels rotated together: a list of (axis, j, first_channel).

    The head dimension is cut into contiguous ranges of d_t, d_h and d_w channels in that order
    (block-diagonal R_3D = diag(R_t, R_y, R_x)); inside a range, pair j is channels
    (off + 2j, off + 2j + 1).  Wan's 44/42/42 gives 22/21/21 pairs.
    """
    pairs = []
    off = 0
    for axis, da in enumerate(split):
        if da % 2 != 0 or da < 0:
            raise ValueError(f"rope range sizes must be even and non-negative, got {split}")
        for j in range(da // 2):
            pairs.append((axis, j, off + 2 * j))
        off += da
    return pairs


def rope_frequencies(split, theta: float = 10000.0):
    """Angular frequency of every pair, per axis: omega_{a,j} = theta^(-2j / d_a).

    Each axis range is an independent 1D RoPE over its own d_a channels ("FLUX's 2D RoPE plus a
    time dimension", first page, "Position: RoPE in three dimensions"); the ladder is a reading,
    pinned in the tests against an independent per-axis implementation.
    """
    return [np.array([theta ** (-2.0 * j / da) for j in range(da // 2)], dtype=np.float64)
            for da in split]


def rope3d_ref(x: np.ndarray, grid, n_text: int = 0, split=(44, 42, 42),
               theta: float = 10000.0, rows=None) -> np.ndarray:
    """Rotate rows of x ([N, heads, d] or [len(rows), heads, d] when ``rows`` is given) by 3D RoPE.

    Pair (x0, x1) of axis a becomes (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi) with
    phi = pos_a * omega_{a,j}; text rows are returned unchanged.  Float64 throughout.
    """
    d = x.shape[-1]
    if sum(split) != d:
        raise ValueError(f"split {split} does not sum to head dim {d}")
    t, h, w, is_video = token_positions(grid, n_text)
    if rows is None:
        rows = np.arange(t.size)
    rows = np.asarray(rows)
    if x.shape[0] != rows.size:
        raise ValueError("x has a different number of rows than selected")
    pos = (t[rows], h[rows], w[rows])
    vid = is_video[rows]
    freqs = rope_frequencies(split, theta)
    y = np.array(x, dtype=ORACLE_DTYPE, copy=True)
    xf = np.asarray(x, dtype=ORACLE_DTYPE)
    for axis, j, c0 in rope_pair_layout(split):
        phi = pos[axis].astype(ORACLE_DTYPE) * freqs[axis][j]
        c = np.where(vid, np.cos(phi), 1.0)[:, None]
        s = np.where(vid, np.sin(phi), 0.0)[:, None]
        x0 = xf[:, :, c0]
        x1 = xf[:, :, c0 + 1]
        y[:, :, c0] = x0 * c - x1 * s
        y[:, :, c0 + 1] = x0 * s + x1 * c
    return y


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------

def attention_dense(qr: np.ndarray, kr: np.ndarray, v: np.ndarray, key_mask=None) -> np.ndarray:
    """Softmax(q k^T / sqrt(d)) v for every query row, one head at a time, in float64.

    Shapes: qr [Nq, heads, d], kr and v [Nk, heads, dv]; ``key_mask`` [Nq, Nk] (True = allowed)
    restricts which keys each query sees.  Non-causal; the softmax subtracts the row maximum.
    """
    d = qr.shape[-1]
    scale = 1.0 / math.sqrt(d)
    nq, heads = qr.shape[0], qr.shape[1]
    out = np.empty((nq, heads, v.shape[-1]), dtype=ORACLE_DTYPE)
    for hd in range(heads):
        s = (np.asarray(qr[:, hd, :], ORACLE_DTYPE) @ np.asarray(kr[:, hd, :], ORACLE_DTYPE).T) * scale
        if key_mask is not None:
            s = np.where(key_mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= p.sum(axis=1, keepdims=True)
        out[:, hd, :] = p @ np.asarray(v[:, hd, :], ORACLE_DTYPE)
    return out


def attention_rows(qr_rows: np.ndarray, kr: np.ndarray, v: np.ndarray, chunk: int = 256) -> np.ndarray:
    """Same result as ``attention_dense`` without a mask, for a subset of query rows.

    ``qr_rows`` [R, heads, d] holds already-rotated query rows; all Nk keys are used.  Query rows
    are processed ``chunk`` at a time so that the score block stays small.
    """
    out = np.empty((qr_rows.shape[0], qr_rows.shape[1], v.shape[-1]), dtype=ORACLE_DTYPE)
    for a in range(0, qr_rows.shape[0], chunk):
        out[a:a + chunk] = attention_dense(qr_rows[a:a + chunk], kr, v)
    return out


def full_attention_ref(q, k, v, grid, n_text: int = 0, split=(44, 42, 42), theta: float = 10000.0,
                       rows=None, heads=None) -> np.ndarray:
    """3D RoPE on q and k, then full non-causal attention over all N = T'H'W' + n_text rows.

    Returns [len(rows), heads, d] (all rows when ``rows`` is None), float64.  ``heads`` optionally
    restricts the computation to a list of head indices (the output then has that many heads).
    """
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    hsel = list(range(q.shape[1])) if heads is None else list(heads)
    out = np.empty((rows.size, len(hsel), v.shape[-1]), dtype=ORACLE_DTYPE)
    for i, hd in enumerate(hsel):
        qh = np.asarray(q[rows, hd:hd + 1, :], ORACLE_DTYPE)
        kh = np.asarray(k[:, hd:hd + 1, :], ORACLE_DTYPE)
        vh = np.asarray(v[:, hd:hd + 1, :], ORACLE_DTYPE)
        qr = rope3d_ref(qh, grid, n_text, split, theta, rows=rows)
        kr = rope3d_ref(kh, grid, n_text, split, theta)
        out[:, i:i + 1, :] = attention_rows(qr, kr, vh)
    return out


def factorized_ref(q, k, v, grid, split=(44, 42, 42), theta: float = 10000.0, rows=None,
                   return_spatial: bool = False):
    """Spatial-then-temporal attention on the same rotated q and k (no text rows).

    Stage 1 (spatial): a query in frame t attends to the S = H'W' keys of frame t, values v.
    Stage 2 (temporal): a query at spatial position s attends to the T' keys at position s in
    every frame, values = stage 1's output.  ``rows`` limits the returned query rows; stage 1 is
    then evaluated at every row stage 2 reads for them.
    """
    t_, h_, w_ = grid
    s_ = h_ * w_
    n = t_ * s_
    if q.shape[0] != n:
        raise ValueError("the factorised path has no text rows: q must have T'H'W' rows")
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    heads = q.shape[1]
    qr_all = rope3d_ref(np.asarray(q, ORACLE_DTYPE), grid, 0, split, theta)
    kr_all = rope3d_ref(np.asarray(k, ORACLE_DTYPE), grid, 0, split, theta)
    vv = np.asarray(v, ORACLE_DTYPE)
    positions = np.unique(rows % s_)
    # stage 1 at every (frame, position) stage 2 needs
    need = np.array(sorted({tt * s_ + int(p) for p in positions for tt in range(t_)}), dtype=np.int64)
    o_s = {}
    for tt in range(t_):
        sel = need[(need // s_) == tt]
        if sel.size == 0:
            continue
        keys = np.arange(tt * s_, (tt + 1) * s_)
        res = attention_dense(qr_all[sel], kr_all[keys], vv[keys])
        for i, r in enumerate(sel):
            o_s[int(r)] = res[i]
    out = np.empty((rows.size, heads, v.shape[-1]), dtype=ORACLE_DTYPE)
    for p in positions:
        seq = np.arange(t_) * s_ + int(p)
        vals = np.stack([o_s[int(x)] for x in seq])
        idx = np.nonzero((rows % s_) == p)[0]
        out[idx] = attention_dense(qr_all[rows[idx]], kr_all[seq], vals)
    if return_spatial:
        return out, o_s
    return out


# --------------------------------------------------------------------------------------------
# Next to the hot path: text cross-attention, partial attention over a run of keys, merge
# --------------------------------------------------------------------------------------------

def cross_attention_ref(q, k, v, rows=None) -> np.ndarray:
    """Video queries against text keys and values: softmax(q k^T / sqrt(d)) v, no rotation.

    q [Nq, heads, d], k and v [Nkv, heads, d]; returns [len(rows), heads, d] in float64.
    """
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows)
    qs = np.asarray(q[rows], ORACLE_DTYPE)
    return attention_rows(qs, np.asarray(k, ORACLE_DTYPE), np.asarray(v, ORACLE_DTYPE))


def partial_attention_ref(q, k, v, grid, n_text: int = 0, split=(44, 42, 42), theta: float = 10000.0,
                          q_begin: int = 0, kv_begin: int = 0):
    """Attention of a run of query rows against a run of key rows, with their global positions.

    q holds global rows [q_begin, q_begin + len(q)), k and v hold rows [kv_begin, kv_begin +
    len(k)) of the same T'H'W' + n_text sequence; each row is rotated by its own (t, h, w).
    Returns (o, lse): o = softmax over this run of keys times v ([len(q), heads, d]) and
    lse = log sum_j exp(s_j / sqrt(d)) over the run ([len(q), heads]), float64.
    """
    q = np.asarray(q, ORACLE_DTYPE)
    k = np.asarray(k, ORACLE_DTYPE)
    v = np.asarray(v, ORACLE_DTYPE)
    qrows = np.arange(q_begin, q_begin + q.shape[0])
    krows = np.arange(kv_begin, kv_begin + k.shape[0])
    qr = rope3d_ref(q, grid, n_text, split, theta, rows=qrows)
    kr = rope3d_ref(k, grid, n_text, split, theta, rows=krows)
    d = q.shape[-1]
    o = np.empty((q.shape[0], q.shape[1], v.shape[-1]), dtype=ORACLE_DTYPE)
    lse = np.empty((q.shape[0], q.shape[1]), dtype=ORACLE_DTYPE)
    for hd in range(q.shape[1]):
        s = (qr[:, hd, :] @ kr[:, hd, :].T) / math.sqrt(d)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        o[:, hd, :] = (e / den) @ v[:, hd, :]
        lse[:, hd] = (m + np.log(den))[:, 0]
    return o, lse


def merge_partials_ref(parts):
    """Combine partial results (o_i, lse_i) over disjoint runs of keys into the result over all.

    lse = log sum_i exp(lse_i) and o = sum_i exp(lse_i - lse) o_i, per row and head.
    """
    lses = np.stack([np.asarray(l, ORACLE_DTYPE) for _, l in parts])          # [P, N, heads]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    o = sum((w[i] / tot)[:, :, None] * np.asarray(parts[i][0], ORACLE_DTYPE) for i in range(len(parts)))
    return o, lse


def qkv_rope_ref(x, w, bias, grid, n_text: int = 0, split=(44, 42, 42), theta: float = 10000.0,
                 heads: int = None, rows=None):
    """QKV projection of x with the 3D rotation of q and k: returns (q~, k~, v), each [rows, heads, d].

    x [N, C], w [3C, C] (output features by input features, rows 0..C-1 give q, C..2C-1 give k,
    2C..3C-1 give v; feature f of a third is channel f % d of head f // d), bias [3C] or None.
    y = x w^T + bias in float64; q and k are then rotated by each row's (t, h, w).
    """
    x = np.asarray(x, ORACLE_DTYPE)
    w = np.asarray(w, ORACLE_DTYPE)
    n, c = x.shape
    if w.shape != (3 * c, c):
        raise ValueError("w must be [3C, C]")
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    d = sum(split)
    if heads is None:
        heads = c // d
    if heads * d != c:
        raise ValueError("C must be heads * d")
    y = x[rows] @ w.T
    if bias is not None:
        y = y + np.asarray(bias, ORACLE_DTYPE)[None, :]
    q = y[:, :c].reshape(rows.size, heads, d)
    k = y[:, c:2 * c].reshape(rows.size, heads, d)
    v = y[:, 2 * c:].reshape(rows.size, heads, d)
    return (rope3d_ref(q, grid, n_text, split, theta, rows=rows),
            rope3d_ref(k, grid, n_text, split, theta, rows=rows), v)


def window_attention_ref(q, k, v, grid, window, split=(44, 42, 42), theta: float = 10000.0, rows=None):
    """Attention inside non-overlapping wt x wh x ww windows of the T' x H' x W' grid (no text).

    Every row is rotated by its own (t, h, w); query row n attends to the rows whose
    (t // wt, h // wh, w // ww) equal its own.  Returns [len(rows), heads, d] in float64.
    """
    t_, h_, w_ = grid
    wt, wh, ww = window
    if t_ % wt or h_ % wh or w_ % ww:
        raise ValueError("window sizes must divide the grid")
    n = t_ * h_ * w_
    if q.shape[0] != n:
        raise ValueError("q must have T'H'W' rows (no text rows)")
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    t, h, w, _ = token_positions(grid)
    win = (t // wt) * ((h_ // wh) * (w_ // ww)) + (h // wh) * (w_ // ww) + (w // ww)
    qr = rope3d_ref(np.asarray(q, ORACLE_DTYPE), grid, 0, split, theta)
    kr = rope3d_ref(np.asarray(k, ORACLE_DTYPE), grid, 0, split, theta)
    vv = np.asarray(v, ORACLE_DTYPE)
    out = np.empty((rows.size, q.shape[1], v.shape[-1]), dtype=ORACLE_DTYPE)
    for wi in np.unique(win[rows]):
        members = np.nonzero(win == wi)[0]
        sel = np.nonzero(win[rows] == wi)[0]
        out[sel] = attention_dense(qr[rows[sel]], kr[members], vv[members])
    return out
