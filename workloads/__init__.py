"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU reference.

This module only draws random numbers and lays out call sequences (which slot a
write starts at, which absolute position its first token has).  It holds none of
the cache arithmetic: no rotary embedding, no quantisation, no attention.  Both
the GPU library and the CPU reference consume exactly the same bytes from here.
"""

from .gen import (  # noqa: F401
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    normal_bf16,
    student_t_outlier_bf16,
    tensor_seed,
    WriteCall,
    steady_ring_schedule,
    tiny_schedule,
    outlier_channels,
    raster_positions,
    CONFIGS,
    ROPE_POSITIONS,
)
