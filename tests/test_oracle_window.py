"""Pins for the oracle's read-time baseline (the linear window the ring replaces), CPU only.

* window_advance against an element-by-element construction, and against the definition of a
  sliding window (after any sequence of advances it holds the last W tokens of the stream);
* the read-time cache equals a ring holding the same tokens in another slot order (one write of
  the same tokens, so the same per-head scales): identical codes slot for slot after the
  permutation, identical attention (non-causal attention does not depend on slot order);
* read-time attention against float64 attention of the unquantised rotated tensors, within the
  FP8 quantisation error.
"""

import math

import numpy as np
import pytest

from oracle import (OracleRing, ring_write, ring_attention, rope_table, window_advance,
                    read_time_ring, read_time_attention)
from oracle.kvcache import softmax_attention, widen_bf16
from oracle.rope import rope_rotate
from workloads import normal_bf16, tensor_seed


@pytest.mark.parametrize("w,n", [(7, 0), (7, 1), (7, 3), (7, 6), (7, 7), (1, 1)])
def test_window_advance_elementwise(w, n):
    rng = np.random.default_rng(w * 10 + n)
    win = rng.integers(0, 1 << 16, size=(w, 2, 3), dtype=np.uint16)
    fresh = rng.integers(0, 1 << 16, size=(n, 2, 3), dtype=np.uint16)
    out = window_advance(win, fresh)
    assert out.shape == win.shape and out.dtype == win.dtype
    for i in range(w):
        want = win[i + n] if i < w - n else fresh[i - (w - n)]
        assert np.array_equal(out[i], want)


def test_window_advance_keeps_the_last_tokens_of_the_stream():
    w = 11
    stream = np.arange(200, dtype=np.int64)[:, None] * 3 + np.arange(3)[None, :]
    win = stream[:w].copy()
    seen = w
    for n in (1, 4, 11, 0, 7, 2, 9, 5):
        win = window_advance(win, stream[seen:seen + n])
        seen += n
        assert np.array_equal(win, stream[seen - w:seen])


def test_window_advance_rejects_bad_shapes():
    with pytest.raises(ValueError):
        window_advance(np.zeros((3, 2)), np.zeros((4, 2)))
    with pytest.raises(ValueError):
        window_advance(np.zeros((3, 2)), np.zeros((1, 3)))


def _window(name, w, h, d):
    return (normal_bf16(tensor_seed(name, 0, 1), (w, h, d)),
            normal_bf16(tensor_seed(name, 0, 2), (w, h, d)))


def test_read_time_cache_equals_a_ring_in_another_slot_order():
    w, h, d, pos0, start = 150, 2, 64, 40, 97
    table = rope_table(pos0 + w, d)
    kw, vw = _window("rt_perm", w, h, d)
    lin = read_time_ring(kw, vw, pos0, table)
    ring = OracleRing(h, w, d)
    ring_write(ring, kw, vw, start, pos0, table)        # token j in slot (start + j) % w
    slots = (start + np.arange(w)) % w
    assert np.array_equal(ring.k[:, slots], lin.k) and np.array_equal(ring.v[:, slots], lin.v)
    assert np.array_equal(ring.k_scale[:, slots], lin.k_scale)
    assert np.array_equal(ring.v_scale[:, slots], lin.v_scale)
    q = normal_bf16(tensor_seed("rt_perm", 1, 0), (20, h, d))
    o1, l1 = read_time_attention(kw, vw, pos0, q, pos0 + w - 20, table, 0.125)
    o2, l2 = ring_attention(ring, start, w, q, pos0 + w - 20, table, 0.125)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def _rotate_f64(x, pos, d):
    """float64 rotation of interleaved pairs at positions pos (independent of the float32 table)."""
    i = np.arange(d // 2)
    ang = pos[:, None].astype(np.float64) * np.power(10000.0, -2.0 * i / d)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def test_read_time_attention_is_exact_attention_up_to_fp8_error():
    w, h, d, pos0, nq = 300, 2, 64, 1000, 40
    table = rope_table(pos0 + w, d)
    kw, vw = _window("rt_exact", w, h, d)
    q = normal_bf16(tensor_seed("rt_exact", 1, 0), (nq, h, d))
    qp = pos0 + w - nq
    o, l = read_time_attention(kw, vw, pos0, q, qp, table, 1 / math.sqrt(d))
    k64 = _rotate_f64(widen_bf16(kw).astype(np.float64), pos0 + np.arange(w), d)
    q64 = _rotate_f64(widen_bf16(q).astype(np.float64), qp + np.arange(nq), d)
    v64 = widen_bf16(vw).astype(np.float64)
    for hh in range(h):
        ro, rl = softmax_attention(q64[:, hh], k64[:, hh], v64[:, hh], 1 / math.sqrt(d))
        rel = np.abs(o[:, hh] - ro).max() / np.abs(ro).max()
        assert rel < 0.08, rel                     # three FP8 roundings (q, k, v): a few percent
        assert np.abs(l[hh] - rl).max() < 0.05
    # a wrong key position (one token off) is far outside that error
    k_off = _rotate_f64(widen_bf16(kw).astype(np.float64), pos0 + 1 + np.arange(w), d)
    ro_off, _ = softmax_attention(q64[:, 0], k_off[:, 0], v64[:, 0], 1 / math.sqrt(d))
    ro0, _ = softmax_attention(q64[:, 0], k64[:, 0], v64[:, 0], 1 / math.sqrt(d))
    assert np.abs(ro_off - ro0).max() / np.abs(ro0).max() > 0.1
