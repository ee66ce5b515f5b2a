"""Write-time FP8 ring KV cache and attention over it, step by step.

Sources (Runway Characters, arXiv 2611.05642):
* abstract -- ring cache; RoPE and FP8 quantisation applied once per write; a delta rotation
  of the cache when positions reset; 757 new-token queries per call against 5,788 slots;
* cpdf.ai blog, section "Como rodar 57B em tempo real com batch size 1" -- instead of
  re-rotating and re-quantising the whole cache at every attention call, both happen as the
  frame enters the cache;
* cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador" -- FP8
  attention with per-head scales.

Readings where the pages are silent (each is repeated where it is used):
* scales are per head and per write: one absmax over the write's n tokens x D channels of a
  head, separately for K (after rotation) and V; every slot a write fills records that
  write's scale, so a ring can hold slots from several writes;
* scale = A/448 and inverse = 448/A with A floored at 2^-100 (so an all-zero head encodes
  to zeros), both correctly rounded float32 divisions; a value x is stored as
  e4m3(x * inverse) and read back as decode(code) * scale;
* the delta rotation dequantises every valid key, rotates it by the position offset, and
  requantises the whole valid ring of a head with one new scale; values are untouched;
* queries are rotated at their own positions and quantised to FP8 with one scale per head
  over all queries of the call (the attention reads FP8 Q, FP8 K and FP8 V);
* attention is non-causal over every valid slot, one KV head per query head, scores
  multiplied by softmax_scale, LSE is the natural log of the softmax denominator plus the
  row maximum; with no valid slot the output is 0 and the LSE is -inf.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode
from .rope import delta_cos_sin, rope_rotate
from .rope3d import delta_cos_sin_3d
from .ring import valid_slots, write_slots

SCALE_FLOOR = np.float32(2.0 ** -100)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class OracleRing:
    """One layer's ring for `heads` heads, in the logical layout: codes [heads, slots, head_dim],
    scales [heads, slots] (float32)."""
    heads: int
    slots: int
    head_dim: int
    k: np.ndarray = field(default=None)
    v: np.ndarray = field(default=None)
    k_scale: np.ndarray = field(default=None)
    v_scale: np.ndarray = field(default=None)

    def __post_init__(self):
        shape = (self.heads, self.slots, self.head_dim)
        if self.k is None:
            self.k = np.zeros(shape, dtype=np.uint8)
        if self.v is None:
            self.v = np.zeros(shape, dtype=np.uint8)
        if self.k_scale is None:
            self.k_scale = np.ones((self.heads, self.slots), dtype=np.float32)
        if self.v_scale is None:
            self.v_scale = np.ones((self.heads, self.slots), dtype=np.float32)

    def copy(self) -> "OracleRing":
        return OracleRing(self.heads, self.slots, self.head_dim, self.k.copy(), self.v.copy(),
                          self.k_scale.copy(), self.v_scale.copy())


def per_head_scale(absmax: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(scale, inverse) per head from the float32 absmax, as float32: A = max(absmax, 2^-100),
    scale = A / 448, inverse = 448 / A."""
    a = np.maximum(np.asarray(absmax, dtype=np.float32), SCALE_FLOOR)
    return (a / np.float32(E4M3_MAX)).astype(np.float32), (np.float32(E4M3_MAX) / a).astype(np.float32)


def quantize_per_head(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x float32 [tokens, heads, D] -> (codes uint8 [tokens, heads, D], scale float32 [heads]).

    One absmax per head over all tokens and channels; codes = e4m3(x * inverse) with the
    float32 product rounded before encoding."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.abs(x).max(axis=(0, 2)) if x.shape[0] > 0 else np.zeros(x.shape[1], np.float32)
    scale, inv = per_head_scale(absmax)
    codes = e4m3_encode((x * inv[None, :, None]).astype(np.float32))
    return codes, scale


def ring_write(ring: OracleRing, k_bits: np.ndarray, v_bits: np.ndarray, start: int, pos0: int,
               table: np.ndarray) -> None:
    """Write n new tokens: K rotated at positions pos0 .. pos0+n-1, K and V quantised with
    per-head scales of this write, stored at slots (start + i) mod S.

    k_bits, v_bits: bfloat16 bit patterns [n, heads, D]; table: float32 [n_pos, D/2, 2]."""
    n = k_bits.shape[0]
    slots = write_slots(start, n, ring.slots)
    pos = pos0 + np.arange(n)
    if pos.min() < 0 or pos.max() >= table.shape[0]:
        raise ValueError("positions outside the rotary table")
    cos = table[pos, :, 0][:, None, :]
    sin = table[pos, :, 1][:, None, :]
    k_rot = rope_rotate(widen_bf16(k_bits), cos, sin)
    kc, ks = quantize_per_head(k_rot)
    vc, vs = quantize_per_head(widen_bf16(v_bits))
    ring.k[:, slots, :] = kc.transpose(1, 0, 2)
    ring.v[:, slots, :] = vc.transpose(1, 0, 2)
    ring.k_scale[:, slots] = ks[:, None]
    ring.v_scale[:, slots] = vs[:, None]


def ring_delta_rotate(ring: OracleRing, head: int, filled: int, delta: int,
                      base: float = 10000.0) -> np.ndarray:
    """Move every valid key by `delta` positions: dequantise (float32 decode * scale), rotate by
    delta, requantise all valid slots of each head with one new per-head scale.

    Returns the float32 rotated keys before requantisation, [heads, filled, D]."""
    c, s = delta_cos_sin(delta, ring.head_dim, base)
    return ring_rotate_by(ring, head, filled, c, s)


def ring_delta_rotate_3d(ring: OracleRing, head: int, filled: int, delta, bands=None,
                         base: float = 10000.0) -> np.ndarray:
    """The same steps for three-axis positions: every valid key moves by the offset triple
    delta = (dt, dy, dx), each band of channel pairs turning by its own coordinate's offset (a
    position reset is (dt, 0, 0)).  Returns the float32 rotated keys before requantisation."""
    c, s = delta_cos_sin_3d(delta, ring.head_dim, bands, base)
    return ring_rotate_by(ring, head, filled, c, s)


def ring_rotate_by(ring: OracleRing, head: int, filled: int, c: np.ndarray,
                   s: np.ndarray) -> np.ndarray:
    """Dequantise every valid key, rotate pair i by the float32 (c[i], s[i]), requantise all
    valid slots of each head with one new per-head scale (V untouched)."""
    vs = valid_slots(head, filled, ring.slots)
    if filled == 0:
        return np.zeros((ring.heads, 0, ring.head_dim), np.float32)
    k = e4m3_decode(ring.k[:, vs, :]).astype(np.float32) * ring.k_scale[:, vs, None]
    k_rot = rope_rotate(k.astype(np.float32), c, s)              # [heads, filled, D]
    codes, scale = quantize_per_head(k_rot.transpose(1, 0, 2))  # tokens first
    ring.k[:, vs, :] = codes.transpose(1, 0, 2)
    ring.k_scale[:, vs] = scale[:, None]
    return k_rot


def q_prep(q_bits: np.ndarray, q_pos0: int, table: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rotate queries at q_pos0 + i and quantise with one scale per head.

    Returns (dequantised Q float64 [nq, heads, D], codes uint8, scale float32 [heads])."""
    nq = q_bits.shape[0]
    pos = q_pos0 + np.arange(nq)
    if nq and (pos.min() < 0 or pos.max() >= table.shape[0]):
        raise ValueError("positions outside the rotary table")
    q_rot = rope_rotate(widen_bf16(q_bits), table[pos, :, 0][:, None, :], table[pos, :, 1][:, None, :])
    codes, scale = quantize_per_head(q_rot)
    q_hat = e4m3_decode(codes) * scale.astype(np.float64)[None, :, None]
    return q_hat, codes, scale


def dequant_ring(ring: OracleRing, head: int, filled: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(valid slots, K_hat, V_hat) with K_hat/V_hat float64 [heads, filled, D] = decode * scale."""
    vs = valid_slots(head, filled, ring.slots)
    k_hat = e4m3_decode(ring.k[:, vs, :]) * ring.k_scale[:, vs, None].astype(np.float64)
    v_hat = e4m3_decode(ring.v[:, vs, :]) * ring.v_scale[:, vs, None].astype(np.float64)
    return vs, k_hat, v_hat


def softmax_attention(q_hat: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                      softmax_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Textbook softmax attention for one head in float64.

    q_hat [nq, D], k_hat/v_hat [n, D] -> (out [nq, D], lse [nq])."""
    nq, d = q_hat.shape
    if k_hat.shape[0] == 0:
        return np.zeros((nq, d)), np.full(nq, -np.inf)
    s = float(softmax_scale) * (q_hat @ k_hat.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v_hat) / l
    return out, (m + np.log(l))[:, 0]


def ring_attention(ring: OracleRing, head: int, filled: int, q_bits: np.ndarray, q_pos0: int,
                   table: np.ndarray, softmax_scale: float,
                   heads: list[int] | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Attention of the nq new queries over every valid slot of the ring.

    Returns (out float64 [nq, heads, D], lse float64 [heads, nq]).  `heads` restricts the
    computation to a subset of heads (others are left as NaN)."""
    q_hat, _, _ = q_prep(q_bits, q_pos0, table)
    _, k_hat, v_hat = dequant_ring(ring, head, filled)
    nq = q_bits.shape[0]
    out = np.full((nq, ring.heads, ring.head_dim), np.nan)
    lse = np.full((ring.heads, nq), np.nan)
    for h in (range(ring.heads) if heads is None else heads):
        out[:, h, :], lse[h] = softmax_attention(q_hat[:, h, :], k_hat[h], v_hat[h],
                                                 float(np.float32(softmax_scale)))
    return out, lse
