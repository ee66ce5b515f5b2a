"""ctypes binding of the C ABI in include/kvring.h (same names, same arguments)."""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libkvring.so")

OP_WRITE, OP_DELTA_ROTATE, OP_ATTENTION, OP_WRITE_ATTEND = 1, 2, 3, 4
TILE = 128
MAX_TOKENS = 16384   # KV_RING_MAX_TOKENS: tokens per write, queries per attention call


class KvRingError(RuntimeError):
    """A C-ABI call returned a negative status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class _Desc(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("heads", ctypes.c_int32),
        ("slots", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it first (python -m fp8_ring_kv_write_amd.build "
            "or __graft_entry__.build()).  There is no fallback path.")
    L = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, f32, f64, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                                  ctypes.c_double, ctypes.c_size_t)
    dp = ctypes.POINTER(_Desc)
    sig = {
        "kv_ring_codes_bytes": (i64, [i32, i32, i32]),
        "kv_ring_k_offset": (i64, [i64, i32, i32]),
        "kv_ring_v_offset": (i64, [i64, i32, i32]),
        "kv_ring_rope_table": (ctypes.c_int, [vp, i64, i32, f64]),
        "kv_ring_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "kv_ring_write": (ctypes.c_int, [dp, vp, vp, i32, i32, i64, vp, i64, vp, sz, vp]),
        "kv_ring_write_static": (ctypes.c_int, [dp, vp, vp, i32, i32, i64, vp, i64, vp]),
        "kv_ring_delta_rotate": (ctypes.c_int, [dp, i32, i32, i64, f64, vp, sz, vp]),
        "kv_ring_rope_table_3d": (ctypes.c_int, [vp, vp, i64, i32, vp, f64]),
        "kv_ring_delta_rotate_3d": (ctypes.c_int, [dp, i32, i32, vp, vp, f64, vp, sz, vp]),
        "ring_attention": (ctypes.c_int, [dp, i32, i32, vp, i32, i64, vp, i64, f32, vp, vp, vp, sz, vp]),
        "kv_ring_fp8_encode": (ctypes.c_int, [vp, vp, i64, vp]),
        "kv_ring_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kv_ring_sync_status": (ctypes.c_int, [vp, vp]),
        "kv_ring_set_attention_events": (ctypes.c_int, [vp, vp]),
        "kv_window_advance": (ctypes.c_int, [vp, vp, vp, i32, i32, i64, vp]),
        "kv_ring_write_attend": (ctypes.c_int, [dp, vp, vp, i32, i32, i64, i32, i32, vp, i32, i64, vp,
                                                i64, f32, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def library_path() -> str:
    return _LIB_PATH


def status_string(status: int) -> str:
    return lib.kv_ring_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvRingError(fn, status)


def codes_bytes(heads: int, slots: int, head_dim: int) -> int:
    return int(lib.kv_ring_codes_bytes(heads, slots, head_dim))


def k_offset(slot: int, channel: int, head_dim: int) -> int:
    """Byte offset of K channel `channel` of slot `slot` within one head's K codes (-1: invalid)."""
    return int(lib.kv_ring_k_offset(slot, channel, head_dim))


def v_offset(slot: int, channel: int, head_dim: int) -> int:
    """Byte offset of V channel `channel` of slot `slot` within one head's V codes (-1: invalid)."""
    return int(lib.kv_ring_v_offset(slot, channel, head_dim))


def rope_table(n_pos: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Host float32 [n_pos, head_dim/2, 2] cos/sin table filled by the library."""
    out = np.empty((n_pos, head_dim // 2, 2), dtype=np.float32)
    _check("kv_ring_rope_table", lib.kv_ring_rope_table(out.ctypes.data, n_pos, head_dim, base))
    return out


def _bands_arg(band_pairs):
    """(int32 array or None, pointer): band pair counts, or NULL for the library's default."""
    if band_pairs is None:
        return None, None
    b = np.ascontiguousarray(np.asarray(band_pairs, dtype=np.int32).reshape(3))
    return b, b.ctypes.data


def rope_table_3d(positions, head_dim: int, band_pairs=None, base: float = 10000.0) -> np.ndarray:
    """Host float32 [n, head_dim/2, 2] cos/sin rows for (frame, row, column) positions [n, 3]."""
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    if pos.ndim != 2 or pos.shape[1] != 3:
        raise ValueError("positions must be [n, 3]")
    out = np.empty((pos.shape[0], head_dim // 2, 2), dtype=np.float32)
    keep, bp = _bands_arg(band_pairs)
    _check("kv_ring_rope_table_3d", lib.kv_ring_rope_table_3d(
        out.ctypes.data, pos.ctypes.data, pos.shape[0], head_dim, bp, base))
    del keep
    return out


def workspace_bytes(op: int, heads: int, slots: int, head_dim: int, n: int) -> int:
    return int(lib.kv_ring_workspace_bytes(op, heads, slots, head_dim, n))


def _stream(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return int(t.data_ptr())


def _same_device(t, device) -> bool:
    d = t.device
    if isinstance(device, str):
        import torch
        device = torch.device(device)
    return d.type == device.type and (device.index is None or d.index == device.index)


def _need(name: str, t, dtype, shape: tuple, device) -> None:
    """Raise ValueError unless tensor t has the dtype, the shape, a contiguous layout and the
    device the call will hand to the library: the kernels read and write exactly that many
    elements at the tensor's address."""
    try:
        ok = t.dtype == dtype
        got = t.shape
    except AttributeError:
        raise ValueError(f"{name}: expected a torch tensor") from None
    if not ok:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if got != shape:
        raise ValueError(f"{name}: shape {tuple(got)}, expected {shape}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: contiguous tensors only")
    if t.device != device and not _same_device(t, device):
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _need_rope(rope, head_dim: int, device) -> None:
    """A rotary table of this head_dim: float32 [n_pos, head_dim/2, 2] or [n_pos, head_dim]."""
    import torch
    try:
        n_pos = rope.shape[0]
        shape = (n_pos, head_dim // 2, 2) if rope.dim() == 3 else (n_pos, head_dim)
    except (AttributeError, IndexError):
        raise ValueError("rope: expected a [n_pos, head_dim/2, 2] float32 tensor") from None
    _need("rope", rope, torch.float32, shape, device)


def _need_workspace(ws, device) -> None:
    if ws is None:
        return
    if not ws.is_contiguous() or not _same_device(ws, device):
        raise ValueError(f"workspace: a contiguous tensor on {device} expected")


class Ring:
    """Device buffers of one ring (one layer, `heads` heads), allocated with torch.

    k, v: uint8 code buffers in the library layout; k_scale, v_scale: float32 [heads, slots].
    Fresh rings hold zero codes and unit scales."""

    def __init__(self, heads: int, slots: int, head_dim: int, device="cuda"):
        import torch
        nbytes = codes_bytes(heads, slots, head_dim)
        if nbytes <= 0:
            raise ValueError("unsupported ring shape")
        self.heads, self.slots, self.head_dim = heads, slots, head_dim
        self.tiles = (slots + TILE - 1) // TILE
        self.device = torch.device(device)
        self.k = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        self.v = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        self.k_scale = torch.ones((heads, slots), dtype=torch.float32, device=self.device)
        self.v_scale = torch.ones((heads, slots), dtype=torch.float32, device=self.device)
        self.device = self.k.device   # with its index (cuda:N), as the tensors handed in report it
        self._desc = _Desc(_ptr(self.k), _ptr(self.v), _ptr(self.k_scale), _ptr(self.v_scale),
                           heads, slots, head_dim)

    @property
    def desc(self):
        return ctypes.byref(self._desc)


# Workspaces of calls made without one: one buffer per (device, stream), kept for the life of
# the process and grown by doubling when a call needs more, so calls do not allocate per shape
# and no buffer is ever released while kernels queued on its stream may still use it (a buffer
# outgrown is kept too).  Calls that share a stream are ordered by it, so they may share its
# buffer; callers that must not allocate at all pass their own workspace.
_WS_POOL: dict = {}
_WS_RETIRED: list = []


def _ws(ws, need: int, device, stream_handle: int):
    import torch
    if ws is not None:
        return ws, int(ws.numel() * ws.element_size())
    dev = torch.device(device)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), int(stream_handle))
    cur = _WS_POOL.get(key)
    if cur is None or cur.numel() < need:
        size = max(need, 1 << 20, 2 * cur.numel() if cur is not None else 0)
        if cur is not None:
            _WS_RETIRED.append(cur)
        # zero-filled: every workspace starts with synchronisation records that must be zero
        # before their first use (every call then leaves them ready for the next)
        cur = torch.zeros(size, dtype=torch.uint8, device=dev)
        _WS_POOL[key] = cur
    return cur, int(cur.numel())


def sync_status(workspace=None, device=None, stream=None) -> int:
    """0 unless a synchronisation wait of the calls made with `workspace` (default: every
    workspace the binding has pooled for `device`) exceeded its bound (then -9: the outputs of
    those calls are not to be trusted, and the workspace must be zero-filled again before further
    use).  Waits for the device first."""
    import torch
    dev = torch.device(device if device is not None else "cuda")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    torch.cuda.synchronize(idx)
    st = _stream(stream, torch.device("cuda", idx))
    if workspace is not None:
        bufs = [workspace]
    else:
        bufs = [b for (d, _), b in _WS_POOL.items() if d == idx]
        bufs += [b for b in _WS_RETIRED if b.device.index == idx]
    for b in bufs:
        r = int(lib.kv_ring_sync_status(_ptr(b), st))
        if r:
            return r
    return 0


def kv_ring_write(ring: Ring, k_new, v_new, start_slot: int, pos0: int, rope, workspace=None,
                  stream=None) -> None:
    """k_new, v_new: bfloat16 [n, heads, head_dim] device tensors; rope: device float32 table."""
    import torch
    n = int(k_new.shape[0])
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(name, t, torch.bfloat16, (n, ring.heads, ring.head_dim), ring.device)
    _need_rope(rope, ring.head_dim, ring.device)
    _need_workspace(workspace, ring.device)
    need = workspace_bytes(OP_WRITE, ring.heads, ring.slots, ring.head_dim, max(n, 1))
    st = _stream(stream, ring.device)
    ws, wsb = _ws(workspace, need, ring.device, st)
    _check("kv_ring_write", lib.kv_ring_write(
        ring.desc, _ptr(k_new), _ptr(v_new), n, start_slot, pos0, _ptr(rope), int(rope.shape[0]),
        _ptr(ws), wsb, st))


def kv_ring_write_static(ring: Ring, k_new, v_new, start_slot: int, pos0: int, rope, stream=None) -> None:
    """kv_ring_write with the library's static scratch instead of a workspace (allocates nothing)."""
    import torch
    n = int(k_new.shape[0])
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(name, t, torch.bfloat16, (n, ring.heads, ring.head_dim), ring.device)
    _need_rope(rope, ring.head_dim, ring.device)
    _check("kv_ring_write_static", lib.kv_ring_write_static(
        ring.desc, _ptr(k_new), _ptr(v_new), n, start_slot, pos0, _ptr(rope), int(rope.shape[0]),
        _stream(stream, ring.device)))


def kv_ring_delta_rotate(ring: Ring, ring_head: int, filled: int, delta: int,
                         rope_base: float = 10000.0, workspace=None, stream=None) -> None:
    _need_workspace(workspace, ring.device)
    need = workspace_bytes(OP_DELTA_ROTATE, ring.heads, ring.slots, ring.head_dim, 0)
    st = _stream(stream, ring.device)
    ws, wsb = _ws(workspace, need, ring.device, st)
    _check("kv_ring_delta_rotate", lib.kv_ring_delta_rotate(
        ring.desc, ring_head, filled, delta, rope_base, _ptr(ws), wsb, st))


def kv_ring_delta_rotate_3d(ring: Ring, ring_head: int, filled: int, delta, band_pairs=None,
                            rope_base: float = 10000.0, workspace=None, stream=None) -> None:
    """Delta rotation by the (frame, row, column) offset triple `delta`."""
    d = np.ascontiguousarray(np.asarray(delta, dtype=np.int64).reshape(3))
    keep, bp = _bands_arg(band_pairs)
    _need_workspace(workspace, ring.device)
    need = workspace_bytes(OP_DELTA_ROTATE, ring.heads, ring.slots, ring.head_dim, 0)
    st = _stream(stream, ring.device)
    ws, wsb = _ws(workspace, need, ring.device, st)
    _check("kv_ring_delta_rotate_3d", lib.kv_ring_delta_rotate_3d(
        ring.desc, ring_head, filled, d.ctypes.data, bp, rope_base, _ptr(ws), wsb, st))
    del keep


def ring_attention(ring: Ring, ring_head: int, filled: int, q, q_pos0: int, rope,
                   softmax_scale: float, out=None, lse=None, workspace=None, stream=None):
    """q: bfloat16 [nq, heads, head_dim].  Returns (out bfloat16 [nq, heads, head_dim],
    lse float32 [heads, nq])."""
    import torch
    nq = int(q.shape[0])
    _need("q", q, torch.bfloat16, (nq, ring.heads, ring.head_dim), ring.device)
    _need_rope(rope, ring.head_dim, ring.device)
    _need_workspace(workspace, ring.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((ring.heads, nq), dtype=torch.float32, device=q.device)
    _need("out", out, torch.bfloat16, (nq, ring.heads, ring.head_dim), ring.device)
    _need("lse", lse, torch.float32, (ring.heads, nq), ring.device)
    need = workspace_bytes(OP_ATTENTION, ring.heads, ring.slots, ring.head_dim, max(nq, 1))
    st = _stream(stream, ring.device)
    ws, wsb = _ws(workspace, need, ring.device, st)
    _check("ring_attention", lib.ring_attention(
        ring.desc, ring_head, filled, _ptr(q), nq, q_pos0, _ptr(rope), int(rope.shape[0]),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), wsb, st))
    return out, lse


def kv_ring_write_attend(ring: Ring, k_new, v_new, start_slot: int, pos0: int, ring_head: int,
                         filled: int, q, q_pos0: int, rope, softmax_scale: float, out=None, lse=None,
                         workspace=None, stream=None):
    """kv_ring_write then ring_attention in one call (ring_head, filled: the ring after the
    write).  Returns (out, lse) like ring_attention."""
    import torch
    n, nq = int(k_new.shape[0]), int(q.shape[0])
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(name, t, torch.bfloat16, (n, ring.heads, ring.head_dim), ring.device)
    _need("q", q, torch.bfloat16, (nq, ring.heads, ring.head_dim), ring.device)
    _need_rope(rope, ring.head_dim, ring.device)
    _need_workspace(workspace, ring.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((ring.heads, nq), dtype=torch.float32, device=q.device)
    _need("out", out, torch.bfloat16, (nq, ring.heads, ring.head_dim), ring.device)
    _need("lse", lse, torch.float32, (ring.heads, nq), ring.device)
    need = workspace_bytes(OP_WRITE_ATTEND, ring.heads, ring.slots, ring.head_dim, max(n, nq, 1))
    st = _stream(stream, ring.device)
    ws, wsb = _ws(workspace, need, ring.device, st)
    _check("kv_ring_write_attend", lib.kv_ring_write_attend(
        ring.desc, _ptr(k_new), _ptr(v_new), n, start_slot, pos0, ring_head, filled, _ptr(q), nq,
        q_pos0, _ptr(rope), int(rope.shape[0]), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
        wsb, st))
    return out, lse


def fp8_encode(x, out=None, stream=None):
    """E4M3 codes of a float32 device tensor with the kernels' encoder."""
    import torch
    _need("x", x, torch.float32, tuple(x.shape), x.device)
    if x.device.type != "cuda":
        raise ValueError("x: a device tensor expected")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need("out", out, torch.uint8, tuple(x.shape), x.device)
    _check("kv_ring_fp8_encode", lib.kv_ring_fp8_encode(_ptr(x), _ptr(out), int(x.numel()),
                                                        _stream(stream, x.device)))
    return out


def kv_window_advance(src, dst, fresh, stream=None) -> None:
    """Read-time baseline copy: dst = src[n:] followed by fresh, for contiguous device tensors of
    rows ([window, ...] and [n, ...] with the same row shape and dtype); dst must not overlap
    src or fresh."""
    window, n = int(dst.shape[0]), int(fresh.shape[0])
    if tuple(src.shape) != tuple(dst.shape) or tuple(fresh.shape[1:]) != tuple(dst.shape[1:]):
        raise ValueError("src, dst and fresh must share the row shape; src and dst the window")
    if src.dtype != dst.dtype or fresh.dtype != dst.dtype:
        raise ValueError("src, dst and fresh must share the dtype")
    if not (src.is_contiguous() and dst.is_contiguous() and fresh.is_contiguous()):
        raise ValueError("contiguous tensors only")
    row_bytes = dst[0].numel() * dst.element_size() if window > 0 else 0
    _check("kv_window_advance", lib.kv_window_advance(
        _ptr(src) if n < window else None, _ptr(dst), _ptr(fresh) if n > 0 else None, window, n,
        row_bytes, _stream(stream, dst.device)))


def set_attention_events(before=None, after=None) -> None:
    """Record torch.cuda.Event `before`/`after` around each later ring_attention call's main
    kernel (both None: off).  The events must have been recorded once through torch (which
    creates the underlying HIP event lazily).  Profiling aid; see include/kvring.h."""
    b = None if before is None else int(before.cuda_event)
    a = None if after is None else int(after.cuda_event)
    if (before is not None or after is not None) and not (a and b):
        raise ValueError("record the events once (event.record()) before handing them over")
    lib.kv_ring_set_attention_events(b if (a and b) else None, a if (a and b) else None)
