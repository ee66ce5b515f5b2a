"""MI355X FP8 ring KV cache: Python binding of libkvring.so.

Argument marshalling only -- every step of the write, the delta rotation and the attention
runs in the HIP kernels behind the C ABI (include/kvring.h).  PyTorch provides device memory
and streams.  Importing this package loads the library and fails loudly when it is missing;
there is no fallback of any kind.
"""

from ._lib import (  # noqa: F401
    KvRingError,
    Ring,
    OP_WRITE,
    OP_DELTA_ROTATE,
    OP_ATTENTION,
    OP_WRITE_ATTEND,
    MAX_TOKENS,
    TILE,
    library_path,
    codes_bytes,
    k_offset,
    v_offset,
    rope_table,
    rope_table_3d,
    workspace_bytes,
    kv_ring_write,
    kv_ring_write_static,
    kv_ring_delta_rotate,
    kv_ring_delta_rotate_3d,
    ring_attention,
    kv_ring_write_attend,
    fp8_encode,
    kv_window_advance,
    set_attention_events,
    status_string,
    sync_status,
    lib,
)
