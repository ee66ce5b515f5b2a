"""CPU oracle for the FP8 ring KV cache: test infrastructure, not part of the product.

A plain, slow, obviously-correct numpy implementation of what the write-time KV-cache
path computes, written from the Runway Characters pages (arXiv 2611.05642):

* abstract: each of the 240 attention calls per chunk reads a 5,788-slot cache of which
  only 757 tokens are new; the whole-cache work is moved to write time -- a ring cache,
  RoPE and FP8 quantisation applied once per write, and a delta rotation when positions
  reset;
* cpdf.ai blog, section "Como rodar 57B em tempo real com batch size 1": rotary positions
  and FP8 quantisation are applied when a frame enters the cache, and the cache is a ring
  so the window advances without copies;
* cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador": the FP8
  attention kernel uses per-head scales.

Where the pages are silent the readings are stated in each function's docstring (pair
layout, RoPE base, FP8 format, scale formula, masking, ...).

Floating point: rotation, scales and quantisation inputs are evaluated in float32 with each
operation rounded on its own (numpy never fuses a multiply with an add); attention is
evaluated in float64.  Everything here is independent of the HIP library: it neither
imports it nor shares any helper, table or constant generator with it.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path never calls it.
"""

from .fp8 import E4M3_MAX, e4m3_decode_table, e4m3_decode, e4m3_encode  # noqa: F401
from .rope import rope_theta, rope_angle, rope_table, rope_rotate  # noqa: F401
from .ring import write_slots, valid_slots, advance  # noqa: F401
from .kvcache import (  # noqa: F401
    OracleRing,
    per_head_scale,
    quantize_per_head,
    ring_write,
    ring_delta_rotate,
    ring_delta_rotate_3d,
    ring_rotate_by,
    q_prep,
    ring_attention,
    SCALE_FLOOR,
)
from .rope3d import default_bands, band_of_pairs, rope_rows_3d, delta_cos_sin_3d  # noqa: F401
from .window import window_advance, read_time_ring, read_time_attention  # noqa: F401
