"""Seeded generators for the synthetic workloads.

The workloads follow the shapes the Runway Characters pages give for one attention
call (abstract of arXiv 2611.05642: a 5,788-slot cache of which 757 tokens are new,
240 calls per chunk; cpdf.ai blog, section "O que a Runway entregou, em numeros":
four denoising passes per chunk).  Head count (24 per GPU), head_dim (128), the
RoPE base, value distributions and absolute positions are not on the pages; the
values here are the stated synthetic stand-ins.

Everything is generated on the host with numpy's PCG64 generator from a seed that
is a stable hash of (workload name, pass, layer, tensor id), then rounded to
bfloat16 (round to nearest even) and handed to both the GPU library and the CPU
reference as the same uint16 bit patterns.
"""

from __future__ import annotations

import hashlib
import struct
from dataclasses import dataclass

import numpy as np

# tensor ids used in seeds
TID_Q, TID_K, TID_V, TID_OUTLIER = 0, 1, 2, 3


def tensor_seed(workload: str, *parts: int) -> int:
    """Stable 64-bit seed from a workload name and integer parts (pass, layer, tensor id, ...)."""
    h = hashlib.blake2b(workload.encode("utf-8"), digest_size=8)
    for p in parts:
        h.update(struct.pack("<q", int(p)))
    return int.from_bytes(h.digest(), "little")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite (the generators never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape) -> np.ndarray:
    """N(0,1) samples rounded to bfloat16, returned as uint16 bit patterns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def outlier_channels(seed: int, heads: int, head_dim: int, frac: float = 0.01) -> np.ndarray:
    """Boolean [heads, head_dim] mask selecting round(frac*heads*head_dim) (head, channel) pairs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    count = int(round(frac * heads * head_dim))
    flat = np.zeros(heads * head_dim, dtype=bool)
    flat[rng.choice(heads * head_dim, size=count, replace=False)] = True
    return flat.reshape(heads, head_dim)


def student_t_outlier_bf16(seed: int, shape, outliers: np.ndarray, nu: float = 3.0,
                           scale: float = 20.0) -> np.ndarray:
    """Student-t(nu) samples of shape [n, heads, head_dim]; the (head, channel) pairs marked in
    `outliers` are multiplied by `scale` for every token.  Rounded to bfloat16 bit patterns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_t(nu, size=shape).astype(np.float32)
    x = np.where(outliers[None, :, :], x * np.float32(scale), x).astype(np.float32)
    return bf16_bits_from_f32(x)


@dataclass(frozen=True)
class WriteCall:
    """One write of `n` new tokens: token i goes to ring slot (start_slot + i) mod slots and has
    absolute position pos0 + i."""
    start_slot: int
    pos0: int
    n: int


def steady_ring_schedule(slots: int = 5788, n: int = 757, writes: int = 8,
                         pos_offset: int = 0) -> list[WriteCall]:
    """Writes that fill a ring to the steady state: chunk c starts where chunk c-1 ended.

    With the default 5,788 slots and 757 tokens, 8 writes (6,056 tokens) fill every slot and the
    last write wraps; the last chunk holds positions pos_offset+5,299 .. pos_offset+6,055."""
    return [WriteCall((n * c) % slots, pos_offset + n * c, n) for c in range(writes)]


def tiny_schedule(slots: int = 64, n: int = 16, writes: int = 6) -> list[WriteCall]:
    """Six writes of 16 tokens into a 64-slot ring (positions 0..95); writes 5 and 6 overwrite
    the oldest slots."""
    return [WriteCall((n * w) % slots, n * w, n) for w in range(writes)]


def raster_positions(n: int, first: int = 0, rows: int = 22, cols: int = 34,
                     t0: int = 0) -> np.ndarray:
    """Synthetic (frame, row, column) positions of tokens first .. first+n-1 of a raster walk
    over frames of rows x cols tokens (column fastest, then row, then frame), the first frame
    being t0: int32 [n, 3].  The default frame of 22 x 34 = 748 tokens is a stand-in for a
    video latent grid; with 757-token chunks the walk runs on into the next frame."""
    i = first + np.arange(n, dtype=np.int64)
    per = rows * cols
    return np.stack([t0 + i // per, (i // cols) % rows, i % cols], axis=1).astype(np.int32)


# The five workloads, as plain data.  Sizes per one GPU's share of heads.
CONFIGS = {
    "tiny": dict(heads=1, head_dim=64, slots=64, n=16, writes=6, rope_base=10000.0,
                 dist="normal"),
    "single_call": dict(heads=24, head_dim=128, slots=5788, nq=757, n=757, writes=8,
                        rope_base=10000.0, dist="normal"),
    "write_path": dict(heads=24, head_dim=128, slots=5788, n=757, start_slot=5500, pos0=12000,
                       rope_base=10000.0, dist="normal"),
    "full_chunk": dict(heads=24, head_dim=128, slots=5788, n=757, passes=4, layers=60,
                       rope_base=10000.0, dist="normal"),
    "reset_outliers": dict(heads=24, head_dim=128, slots=5788, n=757, layers=60, delta=-4000,
                           pos_offset=5944, rope_base=10000.0, dist="student_t3_outliers"),
}

# Positions covered by the rotary table handed to the library (0 .. ROPE_POSITIONS-1).
ROPE_POSITIONS = 16384
