"""Three-axis rotary positions (frame, row, column) for a video cache, and the delta rotation
that moves only the frame axis.

The pages say the cache applies rotary positions when a frame enters it and rotates the cache
by a delta when positions reset (abstract of arXiv 2611.05642; cpdf.ai blog, section "Como
rodar 57B em tempo real com batch size 1"); the model is a video diffusion transformer.  They
give neither the rotary variant nor which axis resets.  Readings for this variant:

* a token's position is a triple (t, y, x): frame, row and column;
* the D/2 interleaved channel pairs are cut into three contiguous bands, frame first, then
  row, then column; each band of P_b pairs is a 1-D rotary embedding of dimension 2 P_b on
  its own coordinate: pair j of the band turns by coordinate * base^(-2j / (2 P_b));
* the default cut gives the row and column bands floor(P/3) pairs each and the frame band the
  rest (P = D/2: 22/21/21 at D = 128, 12/10/10 at D = 64);
* a position reset moves the frame coordinate only: the delta rotation turns the frame band
  by delta_t and the row and column bands by zero, i.e. by cos 0 = 1, sin 0 = 0; it uses
  the same dequantise / rotate / requantise steps as the 1-D delta rotation;
* cos and sin are taken in float64 by the C library (Python's math module) and rounded once
  to float32, as for the 1-D table.

A per-token table of cos/sin rows [n, D/2, 2] is all the write and the attention need: row i
serves token i (the 1-D path indexes its table at pos0 + i, so such a table is used with
position offset 0).

Test infrastructure, like the rest of the oracle.
"""

from __future__ import annotations

import math

import numpy as np


def default_bands(head_dim: int) -> tuple[int, int, int]:
    """(frame, row, column) pairs per band: row and column floor(P/3) each, frame the rest."""
    p = head_dim // 2
    return (p - 2 * (p // 3), p // 3, p // 3)


def _bands(head_dim: int, bands) -> tuple[int, int, int]:
    b = default_bands(head_dim) if bands is None else tuple(int(x) for x in bands)
    if len(b) != 3 or min(b) < 0 or sum(b) != head_dim // 2:
        raise ValueError("bands must be three non-negative pair counts summing to head_dim/2")
    return b


def band_of_pairs(head_dim: int, bands=None) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """For each pair k < D/2: (band index, index j within the band, pairs in that band)."""
    b = _bands(head_dim, bands)
    band = np.repeat(np.arange(3), b)
    local = np.concatenate([np.arange(n) for n in b]).astype(np.int64)
    size = np.repeat(np.asarray(b, dtype=np.int64), b)
    return band, local, size


def _cos_sin_rows(coords: np.ndarray, head_dim: int, bands, base: float) -> np.ndarray:
    """float32 [n, D/2, 2] for integer coordinate triples coords [n, 3]."""
    band, local, size = band_of_pairs(head_dim, bands)
    n = coords.shape[0]
    out = np.empty((n, head_dim // 2, 2), dtype=np.float32)
    for i in range(n):
        for k in range(head_dim // 2):
            theta = math.pow(base, -(2.0 * int(local[k])) / (2 * int(size[k])))
            a = float(int(coords[i, band[k]])) * theta
            out[i, k, 0] = np.float32(math.cos(a))
            out[i, k, 1] = np.float32(math.sin(a))
    return out


def rope_rows_3d(positions: np.ndarray, head_dim: int, bands=None,
                 base: float = 10000.0) -> np.ndarray:
    """cos/sin rows of n tokens at positions [n, 3] = (t, y, x): float32 [n, D/2, 2]."""
    positions = np.asarray(positions)
    if positions.ndim != 2 or positions.shape[1] != 3:
        raise ValueError("positions must be [n, 3]")
    return _cos_sin_rows(positions, head_dim, bands, base)


def delta_cos_sin_3d(delta, head_dim: int, bands=None,
                     base: float = 10000.0) -> tuple[np.ndarray, np.ndarray]:
    """float32 cos/sin [D/2] of the rotation by the offset triple delta = (dt, dy, dx)."""
    rows = _cos_sin_rows(np.asarray(delta, dtype=np.int64).reshape(1, 3), head_dim, bands, base)
    return rows[0, :, 0].copy(), rows[0, :, 1].copy()

