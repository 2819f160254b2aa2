"""Seeded synthetic inputs shared by the oracle side and the HIP side of the tests and the bench.

This module holds no arithmetic of the attention method: it only draws random numbers, rounds them
to the storage type the GPU path reads (bfloat16, round-to-nearest-even, or float32), and picks
which query rows a sampled parity check looks at.  Both the oracle and the device path receive the
exact same stored values from here.

Distribution recipe (no public dataset or trained weights are involved): q, k and v are standard
normal draws from ``numpy.random.Generator(PCG64(seed))`` in float32 with seeds ``base``,
``base + 1`` and ``base + 2``; an optional per-(token, head) row scale drawn from U(lo, hi) with
seed ``base + 4`` multiplies each row of d values before the single rounding to the storage type.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "QKV",
    "make_qkv",
    "sample_rows",
    "sample_rows_per_head",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bits.

    NaN inputs stay NaN (quiet bit set); this is storage conversion only.  Works in chunks of
    uint32 arithmetic (finite values cannot carry out of 32 bits).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    step = 1 << 24
    for a in range(0, flat.size, step):
        u = flat[a:a + step].view(np.uint32)
        nan = np.isnan(flat[a:a + step])
        r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        if nan.any():
            r[nan] = (u[nan] >> np.uint32(16)) | np.uint32(0x40)
        out[a:a + step] = r.astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class QKV:
    """One set of attention inputs of shape [N, heads, d].

    ``dtype`` is "bf16" or "f32".  For "bf16" the ``*_bits`` arrays hold the uint16 bit patterns
    that go to the device and ``q``/``k``/``v`` hold their exact float32 values; for "f32" the
    ``*_bits`` fields are None.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def _normal(seed: int, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal(size=shape, dtype=np.float32)


def make_qkv(n_tokens: int, heads: int, d: int, seed_base: int, dtype: str = "bf16",
             row_scale: tuple[float, float] | None = None, v_offset: float = 0.0,
             q_mult: float = 1.0, k_ramp: float = 0.0) -> QKV:
    """Draw q, k, v ~ N(0, 1) of shape [n_tokens, heads, d].

    ``row_scale=(lo, hi)`` multiplies every (token, head) row of each tensor by an independent
    U(lo, hi) factor before rounding.  ``v_offset`` adds a constant to every v entry and ``q_mult``
    multiplies q, both before rounding (stress variants for normalisation and peaky softmax).
    ``k_ramp`` multiplies k row n by 1 + k_ramp * n / n_tokens, so that scores grow along the
    sequence and a running maximum keeps moving.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    shape = (n_tokens, heads, d)
    tensors = []
    scales = None
    if row_scale is not None:
        g = np.random.Generator(np.random.PCG64(seed_base + 4))
        lo, hi = row_scale
        scales = g.uniform(lo, hi, size=(3, n_tokens, heads, 1)).astype(np.float32)
    for i in range(3):
        x = _normal(seed_base + i, shape)
        if scales is not None:
            x *= scales[i]
        if i == 0 and q_mult != 1.0:
            x *= np.float32(q_mult)
        if i == 2 and v_offset != 0.0:
            x += np.float32(v_offset)
        if i == 1 and k_ramp != 0.0:
            ramp = 1.0 + k_ramp * np.arange(n_tokens, dtype=np.float64) / n_tokens
            x *= ramp.astype(np.float32)[:, None, None]
        tensors.append(x)
    if dtype == "f32":
        return QKV(q=tensors[0], k=tensors[1], v=tensors[2], dtype="f32")
    bits = [f32_to_bf16_bits(x) for x in tensors]
    vals = [bf16_bits_to_f32(b) for b in bits]
    return QKV(q=vals[0], k=vals[1], v=vals[2], dtype="bf16",
               q_bits=bits[0], k_bits=bits[1], v_bits=bits[2])


def sample_rows(n_tokens: int, n_video: int, tokens_per_frame: int, n_samples: int, seed: int,
                tile_rows: int = 256) -> np.ndarray:
    """Choose the query rows a sampled check compares, sorted and without repeats.

    Edge rows come first (row 0, 1, the last row of the first frame, the first row of the
    second frame, the last video row, the last row overall, the first row of the last query tile
    of ``tile_rows`` rows, the middle row); the rest are drawn without replacement from
    ``numpy.random.Generator(PCG64(seed))``.  If ``n_samples >= n_tokens`` every row is returned.
    """
    if n_samples >= n_tokens:
        return np.arange(n_tokens, dtype=np.int64)
    forced = [0, 1, tokens_per_frame - 1, tokens_per_frame, n_video - 1, n_tokens - 1,
              ((n_tokens - 1) // tile_rows) * tile_rows, n_tokens // 2]
    chosen = []
    for r in forced:
        if 0 <= r < n_tokens and r not in chosen:
            chosen.append(int(r))
    g = np.random.Generator(np.random.PCG64(seed))
    rest = np.setdiff1d(np.arange(n_tokens, dtype=np.int64), np.array(chosen, dtype=np.int64))
    need = max(0, min(n_samples - len(chosen), rest.size))
    extra = g.choice(rest, size=need, replace=False)
    return np.sort(np.concatenate([np.array(chosen, dtype=np.int64), extra.astype(np.int64)]))


def sample_rows_per_head(n_tokens: int, n_video: int, tokens_per_frame: int, n_samples: int,
                         seed: int, head: int, tile_rows: int = 256) -> np.ndarray:
    """The rows checked for one head: ``sample_rows`` with the seed ``seed + head``, so that each
    head is compared on its own draw (the edge rows are in every head's set)."""
    return sample_rows(n_tokens, n_video, tokens_per_frame, n_samples, seed + head, tile_rows)
