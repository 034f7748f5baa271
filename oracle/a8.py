"""INT8-activation variant of the projections (oracle; test infrastructure only).

"How To Build Your Own LLM Runtime From Scratch" (daily.dev), Summary and the
FAQ question on FP16-activation INT4 unpacking against INT8-activation dp4a:
the build quantised the fp16 activations to INT8 in an extra kernel before
each GEMV and multiplied them with the INT4 weights in integer arithmetic;
that path was benchmarked and removed. The pages give no quantisation rule.
The reading taken here (READING) mirrors the weight rule of ``quant.py``:
symmetric, one scale per row and group of 128 consecutive inputs (the weight
groups), so that each group's product is an exact integer sum:

  a  = max |x| over the group                 (float32, exact)
  s  = float32(a / 127)
  q  = clamp( round_half_even( float32(x) / s ), -127, 127 ),  q = 0 if s == 0
  y[b][n] = sum_g  sw[n][g] * s[b][g] * sum_{k in g} qw[n][k] * q[b][k]

The activation quantiser is defined in binary32 throughout (READING): its
scale is itself a binary32 quotient, fl32(fl32(max|x|) / 127), and the code
decision is the correctly rounded binary32 quotient of the two binary32
operands fl32(x) and s, rounded half to even. (The weight rule of
``quant.py`` takes its quotient in binary64 because its scale is an fp16
number and exact ties of w / s16 must reach round-half-even intact.) A
binary64 quotient would decide differently only when the exact quotient lies
within half a binary32 ulp of a tie; tests/golden/a8_hand.json pins one such
case (x = max / 2). The products and sums after the decision are float64.
"""
from __future__ import annotations

import numpy as np

from .quant import GROUP

F16 = np.float16
F32 = np.float32
F64 = np.float64


def quantize_a8(x16, group: int = GROUP):
    """Quantise fp16 activations ``x16`` [..., K] per row and group of ``group``.

    Returns ``(q, s)``: int8 codes [..., K] in [-127, 127] and float32 scales
    [..., K // group]."""
    x = np.asarray(x16, dtype=F16).astype(F32)
    *lead, k = x.shape
    if k % group != 0:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    xg = x.reshape(*lead, k // group, group)
    a = np.max(np.abs(xg), axis=-1)                                   # float32, exact
    s = (a / F32(127.0)).astype(F32)
    r = np.zeros_like(xg)
    np.divide(xg, s[..., None], out=r, where=(s[..., None] != 0))     # float32 quotient
    q = np.clip(np.rint(r), -127, 127).astype(np.int8)
    return q.reshape(x.shape), s


def dequantize_a8(q, s, group: int = GROUP) -> np.ndarray:
    """x^[..., k] = q[..., k] * s[..., k // group] (float64, exact)."""
    q = np.asarray(q)
    return q.astype(F64) * np.repeat(np.asarray(s, F32).astype(F64), group, axis=-1)


def gemv_w4a8(qw, sw16, qx, sx, bias16=None, group: int = GROUP) -> np.ndarray:
    """y [B, N] (float64) of INT4 weights (codes ``qw`` [N, K], fp16 scales
    ``sw16`` [N, K/group]) times INT8 activations (``qx`` [B, K], float32
    scales ``sx`` [B, K/group]). Each group's sum of code products is an exact
    integer (|q_w q_x| <= 1016, 128 terms: exact in float64)."""
    qw = np.asarray(qw)
    qx = np.atleast_2d(np.asarray(qx))
    n, k = qw.shape
    G = k // group
    sw = np.asarray(sw16, F16).astype(F64)
    sxx = np.atleast_2d(np.asarray(sx, F32)).astype(F64)
    y = np.zeros((qx.shape[0], n), F64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        dots = qx[:, sl].astype(F64) @ qw[:, sl].astype(F64).T          # exact integers
        y += dots * sxx[:, g:g + 1] * sw[None, :, g]
    if bias16 is not None:
        y = y + np.asarray(bias16, F16).astype(F64)
    return y
