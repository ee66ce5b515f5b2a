"""Rotary position embedding as the write-time cache applies it.

The pages say rotary positions are applied once, when a frame enters the cache, and that
positions that reset are handled by a delta rotation (abstract of arXiv 2611.05642; cpdf.ai
blog, section "Como rodar 57B em tempo real com batch size 1").  They do not give the
variant.  Readings:

* 1-D positions, base 10000 unless stated, head_dim D even;
* pairs are interleaved channels (2i, 2i+1), i < D/2, with frequency
  theta_i = base^(-2i/D) radians per position;
* the pair (x, y) at position p is treated as the complex number x + iy and multiplied by
  exp(i p theta_i):  x' = x cos - y sin,  y' = x sin + y cos.  Because exp(i p t) exp(i d t)
  = exp(i (p+d) t), rotating a key already at position p by d moves it to position p + d,
  which is what the delta rotation relies on;
* cos and sin are evaluated in float64 by the C library (through Python's math module) on
  the float64 angle p * theta_i and rounded once to float32; the rotation itself is four
  float32 products and two float32 sums, each rounded on its own (no fused multiply-add).
"""

from __future__ import annotations

import functools
import math

import numpy as np


def rope_theta(i: int, head_dim: int, base: float = 10000.0) -> float:
    """Frequency of pair i in radians per position (float64)."""
    return math.pow(base, -(2.0 * i) / head_dim)


def rope_angle(p: int, i: int, head_dim: int, base: float = 10000.0) -> float:
    """Angle of pair i at (possibly negative) position offset p, in float64."""
    return float(p) * rope_theta(i, head_dim, base)


def _cos_sin_f32(p: int, head_dim: int, base: float) -> tuple[np.ndarray, np.ndarray]:
    c = np.empty(head_dim // 2, dtype=np.float32)
    s = np.empty(head_dim // 2, dtype=np.float32)
    for i in range(head_dim // 2):
        a = rope_angle(p, i, head_dim, base)
        c[i] = np.float32(math.cos(a))
        s[i] = np.float32(math.sin(a))
    return c, s


@functools.lru_cache(maxsize=8)
def rope_table(n_pos: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 [n_pos, head_dim/2, 2] table: [p, i, 0] = cos(p theta_i), [p, i, 1] = sin(p theta_i)."""
    t = np.empty((n_pos, head_dim // 2, 2), dtype=np.float32)
    for p in range(n_pos):
        c, s = _cos_sin_f32(p, head_dim, base)
        t[p, :, 0] = c
        t[p, :, 1] = s
    t.setflags(write=False)
    return t


def delta_cos_sin(delta: int, head_dim: int, base: float = 10000.0) -> tuple[np.ndarray, np.ndarray]:
    """float32 cos/sin of delta * theta_i for the delta rotation (delta may be negative)."""
    return _cos_sin_f32(delta, head_dim, base)


def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate float32 x[..., D] pairwise by float32 cos/sin[..., D/2] (broadcast), in float32."""
    x = np.asarray(x, dtype=np.float32)
    cos = np.asarray(cos, dtype=np.float32)
    sin = np.asarray(sin, dtype=np.float32)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = (xe * cos) - (xo * sin)
    out[..., 1::2] = (xe * sin) + (xo * cos)
    return out
