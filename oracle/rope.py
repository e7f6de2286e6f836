"""Rotary position embedding in float64.  (Oracle: test infrastructure only.)

[P1] "what to keep, how to align positions" (§3.3): RoPE encodes a token's
position by cosine/sine rotations; moving a cached key from position p to q
multiplies it by a rotation matrix and leaves the value alone.  The displayed
equation was lost, so the standard per-pair rotation is used (a reading):

    theta_i = base ** (-2 i / d),             i = 0 .. d/2-1
    pair i of x  = (x[i], x[i + d/2])          layout "half"   (default)
                 = (x[2i], x[2i+1])            layout "interleaved"
    RoPE(x, p)   rotates pair i by the angle p * theta_i:
                 (a, b) -> (a cos - b sin, a sin + b cos)

Rotation p -> q is RoPE(., q - p).  The angle is the exact integer position
times the fp64 frequency; numpy's cos/sin do their own argument reduction.
"""
from __future__ import annotations

import numpy as np

HALF, INTERLEAVED = 0, 1


def theta(d: int, base: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def _pairs(d, layout):
    if layout == HALF:
        a = np.arange(d // 2)
        return a, a + d // 2
    if layout == INTERLEAVED:
        a = np.arange(0, d, 2)
        return a, a + 1
    raise ValueError(layout)


def rope(x, pos, base: float = 150000.0, layout: int = HALF) -> np.ndarray:
    """Rotate x[..., d] to position `pos` (integer array broadcast against
    x.shape[:-1], or against its leading axis when pos is 1-D)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.asarray(pos, dtype=np.int64)
    if pos.ndim == 1 and x.ndim > 1:
        pos = pos.reshape(pos.shape + (1,) * (x.ndim - 2))
    ang = pos.astype(np.float64)[..., None] * theta(d, base)  # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    ia, ib = _pairs(d, layout)
    a, b = x[..., ia], x[..., ib]
    out = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (d,)), np.float64)
    out[..., ia] = a * c - b * s
    out[..., ib] = a * s + b * c
    return out


def rotate(x, pos_from, pos_to, base: float = 150000.0, layout: int = HALF) -> np.ndarray:
    """Move keys from position pos_from to pos_to: R((pos_to - pos_from) theta) x."""
    return rope(x, np.asarray(pos_to, np.int64) - np.asarray(pos_from, np.int64), base, layout)
