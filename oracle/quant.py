"""Symmetric group-wise INT4 quantisation (oracle; test infrastructure only).

Follows "How to build your own LLM runtime from scratch", section "What it
actually builds": INT4 weights, symmetric (no zero point), one scale per group
of 128 consecutive weights. The pages do not print the scale rule; the reading
taken here (READING) is the one that makes the round-trip error at most half a
scale step for every weight:

  a    = max |w| over the group (float32, exact)
  s16  = float16_RNE( float32(a / 7) )
  q    = clamp( round_half_even( float64(w) / float64(s16) ), -8, 7 ),  q = 0 if s16 == 0
  w^   = q * s16

Dividing by 7 (not 8) keeps +a representable (a/s16 <= 7.004 -> 7), so the
codes actually used lie in [-7, 7]. The quotient is taken in float64 so that
exact ties are decided by round-half-even.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def quantize_w4(w: np.ndarray, group: int = GROUP):
    """Quantise float32 ``w`` [N, K] along K in groups of ``group``.

    Returns ``(q, s16)``: int8 codes [N, K] in [-8, 7] and float16 scales
    [N, K // group].
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if k % group != 0:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    wg = w.reshape(n, k // group, group)
    a = np.max(np.abs(wg), axis=2)                       # float32, exact
    s16 = (a / np.float32(7.0)).astype(np.float32).astype(np.float16)
    if np.any(np.isinf(s16)):
        raise ValueError("group scale overflows float16")
    sd = s16.astype(np.float64)[:, :, None]
    num = wg.astype(np.float64)
    r = np.zeros_like(num)
    np.divide(num, sd, out=r, where=(sd != 0))
    q = np.clip(np.rint(r), -8, 7).astype(np.int8)
    return q.reshape(n, k), s16


def dequantize_w4(q: np.ndarray, s16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """w^[n, k] = q[n, k] * s16[n, k // group], in float64 (exact)."""
    q = np.asarray(q)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    n, k = q.shape
    if s.shape != (n, k // group):
        raise ValueError("scale shape does not match codes")
    return q.astype(np.float64) * np.repeat(s, group, axis=1)
