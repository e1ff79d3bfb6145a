"""Counter-based dropout mask of the float64 oracle (TEST INFRASTRUCTURE ONLY).

Page "python-20261012-ragged-flash-attention-gradient-recompute", section
"Root causes addressed": dropout draws its randomness from a counter-based
splitmix64 hash of (seed, b, h, row, col), so the backward rebuilds exactly
the forward's mask whatever the tiling, with one rate for everything or one
per row.  The pages fix neither how the five values are combined nor how a
word becomes a keep decision; the reading taken:

* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", 2014): from state x it returns mix64(x + n * gamma) as its
  n-th output (n = 1, 2, ...), gamma = 0x9E3779B97F4A7C15, and mix64 is its
  output function (xor-shift 30, multiply, xor-shift 27, multiply,
  xor-shift 31), all modulo 2^64;
* the (sequence b, query head h) pair owns the stream whose state is output
  number b * 2^16 + h + 1 of the generator started at `seed`;
* the word of local query row i and local key j is output number
  i * 2^32 + j + 1 of that stream;
* with rate p (float32, 0 <= p < 1) the threshold is T = floor(p * 2^32),
  computed exactly; key j of row i is kept iff (word >> 32) >= T, and a kept
  weight is scaled by 1 / (1 - p).  A per-row rate [tokens, heads] gives each
  (token, head) row its own T and scale.

Only the mask and the scale come from here; attention.py applies them.
"""
from __future__ import annotations

import numpy as np

__all__ = ["GAMMA", "mix64", "splitmix64_outputs", "stream_state", "words", "threshold",
           "keep_scale"]

GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)


def mix64(z):
    """splitmix64's output function on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
    return z ^ (z >> np.uint64(31))


def splitmix64_outputs(state: int, n: int) -> list:
    """The first n outputs of the generator started at `state`, stepped one
    at a time (plain Python integers)."""
    out = []
    x = state & _M64
    for _ in range(n):
        x = (x + GAMMA) & _M64
        out.append(int(mix64(np.uint64(x))))
    return out


def stream_state(seed: int, b: int, h: int) -> int:
    """State of the (sequence, head) stream: output b * 2^16 + h + 1 of the
    generator started at `seed`."""
    n = (int(b) << 16) + int(h) + 1
    return int(mix64(np.uint64((int(seed) + n * GAMMA) & _M64)))


def words(seed: int, b: int, h: int, i_pos, Lk: int):
    """uint64 [n, Lk]: output i * 2^32 + j + 1 of the (b, h) stream for each
    local row i in i_pos and key j < Lk."""
    s = stream_state(seed, b, h)
    i_pos = np.asarray(i_pos, dtype=np.uint64)
    j = np.arange(Lk, dtype=np.uint64)
    with np.errstate(over="ignore"):
        n = (i_pos[:, None] << np.uint64(32)) + j[None, :] + np.uint64(1)
        return mix64(np.uint64(s) + n * np.uint64(GAMMA))


def threshold(rate) -> np.ndarray:
    """floor(p * 2^32) of float32 rates p in [0, 1), as uint64 (exact)."""
    p = np.asarray(rate, dtype=np.float32).astype(np.float64)
    if np.any(p < 0.0) or np.any(p >= 1.0):
        raise ValueError("dropout rates must lie in [0, 1)")
    return np.floor(p * 4294967296.0).astype(np.uint64)


def keep_scale(seed: int, b: int, h: int, i_pos, Lk: int, rates):
    """float64 [n, Lk]: 1 / (1 - p_i) where key j of row i is kept, else 0.
    `rates` holds the float32 rate of each row (length n)."""
    rates = np.asarray(rates, dtype=np.float32)
    T = threshold(rates)
    keep = (words(seed, b, h, i_pos, Lk) >> np.uint64(32)) >= T[:, None]
    scale = 1.0 / (1.0 - rates.astype(np.float64))
    return np.where(keep, scale[:, None], 0.0)
