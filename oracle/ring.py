"""Ring slot bookkeeping.

The cache is a ring of a fixed number of slots per layer so that the attention window
advances without copying (abstract of arXiv 2611.05642; cpdf.ai blog, section "Como rodar
57B em tempo real com batch size 1").  Readings (the pages give no indexing):

* a write of n tokens starting at slot `start` puts token i in slot (start + i) mod S;
* the caller keeps `head` (the slot after the newest token) and `filled` (how many slots
  hold tokens); after a write head = (start + n) mod S and filled = min(filled + n, S);
* the valid slots are the `filled` slots just before `head`, oldest first:
  (head - filled + j) mod S for j in 0 .. filled-1.
"""

from __future__ import annotations

import numpy as np


def write_slots(start: int, n: int, slots: int) -> np.ndarray:
    """Slot of each of the n new tokens."""
    if not (0 <= start < slots) or not (1 <= n <= slots):
        raise ValueError("need 0 <= start < slots and 1 <= n <= slots")
    return (start + np.arange(n, dtype=np.int64)) % slots


def valid_slots(head: int, filled: int, slots: int) -> np.ndarray:
    """Slots holding tokens, oldest first."""
    if not (0 <= head < slots) or not (0 <= filled <= slots):
        raise ValueError("need 0 <= head < slots and 0 <= filled <= slots")
    return (head - filled + np.arange(filled, dtype=np.int64)) % slots


def advance(start: int, n: int, filled: int, slots: int) -> tuple[int, int]:
    """(head, filled) after a write of n tokens at `start`."""
    return (start + n) % slots, min(filled + n, slots)
