"""Read-time baseline: the linear cache window that the ring replaces.

Before the change the Runway Characters pages describe (abstract of arXiv 2611.05642: the
whole-cache work repeated in each of the 240 attention calls is moved to write time; cpdf.ai
blog, section "Como rodar 57B em tempo real com batch size 1": the ring lets the window advance
without copies), every call worked on the whole cache:

1. the window of the last W tokens (bfloat16, unrotated) is advanced by copying: the oldest n
   tokens drop out, the n new ones are appended;
2. the whole window is rotated at its positions and quantised to FP8 again, here read as one
   write of all W tokens (one scale per head over the window) into a ring of W slots starting
   at slot 0;
3. the attention reads that cache: valid slots 0 .. W-1, ring head 0.

Test infrastructure, like the rest of the oracle.
"""

from __future__ import annotations

import numpy as np

from .kvcache import OracleRing, ring_write, ring_attention


def window_advance(window: np.ndarray, fresh: np.ndarray) -> np.ndarray:
    """The window after n = len(fresh) new tokens: rows n.. of the old window, then the new
    rows (any row shape and dtype)."""
    n, w = fresh.shape[0], window.shape[0]
    if n > w or window.shape[1:] != fresh.shape[1:]:
        raise ValueError("need n <= window and matching row shapes")
    return np.concatenate([window[n:], fresh], axis=0)


def read_time_ring(k_window: np.ndarray, v_window: np.ndarray, pos0: int,
                   table: np.ndarray) -> OracleRing:
    """Step 2: the whole window (token j at position pos0 + j) rotated and quantised as one write
    into a fresh ring of W slots at slot 0."""
    w, heads, d = k_window.shape
    ring = OracleRing(heads, w, d)
    ring_write(ring, k_window, v_window, 0, pos0, table)
    return ring


def read_time_attention(k_window: np.ndarray, v_window: np.ndarray, pos0: int, q_bits: np.ndarray,
                        q_pos0: int, table: np.ndarray, softmax_scale: float, heads=None):
    """Steps 2 and 3 for one call: attention of the queries over the requantised window."""
    ring = read_time_ring(k_window, v_window, pos0, table)
    return ring_attention(ring, 0, ring.slots, q_bits, q_pos0, table, softmax_scale, heads=heads)
