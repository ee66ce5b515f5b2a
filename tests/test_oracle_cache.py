"""Pins for the oracle's write, delta rotation, query preparation and attention (CPU only).

What pins what:
* attention: a pure-Python double loop with math.exp on tiny inputs, torch's
  scaled_dot_product_attention in float64, and closed forms (one valid slot; zero query);
* write-time cache == read-time cache: a plain linear window that keeps the bfloat16 tokens
  and rotates/quantises at read time gives the same dequantised keys and values;
* delta rotation: equals re-rotation at the shifted positions up to the FP8 error of the
  first write; +delta then -delta is the identity up to float32 rounding; delta = 0 leaves
  the codes unchanged; attention is invariant when queries and keys move together.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (OracleRing, e4m3_decode, e4m3_encode, q_prep, ring_attention, ring_delta_rotate,
                    ring_write, rope_rotate, rope_table, valid_slots, advance, per_head_scale)
from oracle.kvcache import dequant_ring, softmax_attention, widen_bf16
from workloads import normal_bf16, tiny_schedule, steady_ring_schedule, tensor_seed


def _tokens(seed, n, h, d):
    return normal_bf16(seed, (n, h, d))


def _fill(ring, schedule, table, name="t"):
    head, filled = 0, 0
    for w in schedule:
        k = _tokens(tensor_seed(name, w.pos0, 1), w.n, ring.heads, ring.head_dim)
        v = _tokens(tensor_seed(name, w.pos0, 2), w.n, ring.heads, ring.head_dim)
        ring_write(ring, k, v, w.start_slot, w.pos0, table)
        head, filled = advance(w.start_slot, w.n, filled, ring.slots)
    return head, filled


# ---------------------------------------------------------------- attention core

def _naive_attention(q, k, v, scale):
    out = []
    lse = []
    for qi in q:
        s = [scale * sum(float(a) * float(b) for a, b in zip(qi, kj)) for kj in k]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        out.append([sum(w[j] * float(v[j][c]) for j in range(len(k))) / tot for c in range(len(qi))])
        lse.append(m + math.log(tot))
    return np.array(out), np.array(lse)


def test_softmax_attention_matches_naive_loop():
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((9, 8)), rng.standard_normal((9, 8))
    o, l = softmax_attention(q, k, v, 0.3)
    o2, l2 = _naive_attention(q, k, v, 0.3)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(l, l2, rtol=1e-12, atol=1e-13)


def test_softmax_attention_matches_torch_sdpa_float64():
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((33, 64)), rng.standard_normal((70, 64)), rng.standard_normal((70, 64))
    o, _ = softmax_attention(q, k, v, 1 / 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=1 / 8)[0].numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_closed_forms_on_ring():
    table = rope_table(128, 64)
    ring = OracleRing(1, 64, 64)
    w = tiny_schedule()[0]
    _fill(ring, [w], table)
    # one valid slot (head = 1, filled = 1 -> slot 0): output is that slot's V_hat exactly
    q = _tokens(5, 3, 1, 64)
    out, lse = ring_attention(ring, 1, 1, q, 16, table, 0.125)
    _, k_hat, v_hat = dequant_ring(ring, 1, 1)
    q_hat, _, _ = q_prep(q, 16, table)
    assert np.array_equal(out[:, 0, :], np.repeat(v_hat[0], 3, axis=0))
    assert np.allclose(lse[0], 0.125 * (q_hat[:, 0, :] @ k_hat[0, 0]), rtol=1e-14, atol=1e-14)
    # zero queries: uniform softmax -> mean of the valid V_hat, lse = ln(filled)
    qz = np.zeros((2, 1, 64), np.uint16)
    out, lse = ring_attention(ring, 16, 16, qz, 0, table, 0.125)
    _, _, v_hat = dequant_ring(ring, 16, 16)
    assert np.allclose(out[:, 0, :], v_hat[0].mean(axis=0)[None], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, math.log(16), rtol=1e-14)
    # no valid slot
    out, lse = ring_attention(ring, 0, 0, q, 16, table, 0.125)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_attention_invariant_to_slot_permutation_and_ignores_unfilled_slots():
    table = rope_table(256, 64)
    ring = OracleRing(2, 64, 64)
    head, filled = _fill(ring, tiny_schedule()[:3], table)   # 48 of 64 slots filled
    q = _tokens(9, 16, 2, 64)
    ref_out, ref_lse = ring_attention(ring, head, filled, q, 32, table, 0.125)
    # poison every unfilled slot: NaN codes and NaN scales must not reach the output
    poisoned = ring.copy()
    free = np.setdiff1d(np.arange(64), valid_slots(head, filled, 64))
    poisoned.k[:, free, :] = 0x7F
    poisoned.v[:, free, :] = 0xFF
    poisoned.k_scale[:, free] = np.nan
    poisoned.v_scale[:, free] = np.nan
    out, lse = ring_attention(poisoned, head, filled, q, 32, table, 0.125)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
    # rotate the ring by 10 slots (same tokens, other slots): same attention
    shifted = OracleRing(2, 64, 64)
    perm = (np.arange(64) + 10) % 64
    shifted.k[:, perm], shifted.v[:, perm] = ring.k, ring.v
    shifted.k_scale[:, perm], shifted.v_scale[:, perm] = ring.k_scale, ring.v_scale
    out2, lse2 = ring_attention(shifted, (head + 10) % 64, filled, q, 32, table, 0.125)
    assert np.allclose(out2, ref_out, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse2, ref_lse, rtol=1e-12)


# ---------------------------------------------------------------- write-time == read-time

def test_write_time_cache_equals_read_time_window():
    """The paper's move: rotating and quantising once at write time gives the same cache
    contents as keeping raw tokens in a sliding window and doing both at every read."""
    S, H, D = 64, 2, 64
    table = rope_table(256, D)
    sched = tiny_schedule()
    raw = [(_tokens(tensor_seed("rt", wid, 1), w.n, H, D), _tokens(tensor_seed("rt", wid, 2), w.n, H, D))
           for wid, w in enumerate(sched)]
    ring = OracleRing(H, S, D)
    window = []   # (write id, index in write), oldest first, at most S entries
    filled = 0
    for wid, w in enumerate(sched):
        ring_write(ring, raw[wid][0], raw[wid][1], w.start_slot, w.pos0, table)
        head, filled = advance(w.start_slot, w.n, filled, S)
        window = (window + [(wid, i) for i in range(w.n)])[-S:]
        _, k_hat, v_hat = dequant_ring(ring, head, filled)
        # read time: for each write still in the window, rotate its raw keys at their
        # positions, take that write's per-head scale, quantise and dequantise
        for j, (wj, i) in enumerate(window):
            p0, n = sched[wj].pos0, sched[wj].n
            krot = rope_rotate(widen_bf16(raw[wj][0]), table[p0:p0 + n, :, 0][:, None],
                               table[p0:p0 + n, :, 1][:, None])
            for x, got in ((krot, k_hat), (widen_bf16(raw[wj][1]), v_hat)):
                sc, inv = per_head_scale(np.abs(x).max(axis=(0, 2)))
                deq = e4m3_decode(e4m3_encode(x[i] * inv[:, None])) * sc.astype(np.float64)[:, None]
                assert np.array_equal(got[:, j, :], deq), (wid, j)


# ---------------------------------------------------------------- delta rotation

def _steady_small(H=2, D=64, S=256, n=48, writes=7, pos_offset=300):
    table = rope_table(1024, D)
    ring = OracleRing(H, S, D)
    sched = steady_ring_schedule(S, n, writes, pos_offset)
    head, filled = _fill(ring, sched, table, "dr")
    return ring, head, filled, table, sched


def test_delta_rotation_equals_rerotation_at_shifted_positions():
    ring, head, filled, table, sched = _steady_small()
    delta = -250
    before = ring.copy()
    k_rot = ring_delta_rotate(ring, head, filled, delta)
    # rebuild raw keys of the valid slots with their original positions
    vs = valid_slots(head, filled, ring.slots)
    raw = np.zeros((ring.heads, ring.slots, ring.head_dim), np.float32)
    pos = np.zeros(ring.slots, np.int64)
    for w in sched:
        k = widen_bf16(_tokens(tensor_seed("dr", w.pos0, 1), w.n, ring.heads, ring.head_dim))
        s = (w.start_slot + np.arange(w.n)) % ring.slots
        raw[:, s, :] = k.transpose(1, 0, 2)
        pos[s] = w.pos0 + np.arange(w.n)
    newpos = pos[vs] + delta
    ref = rope_rotate(raw[:, vs, :], table[newpos, :, 0][None], table[newpos, :, 1][None])
    # error budget: one FP8 rounding of the first write (half an ulp: 2^-4 relative, at most
    # 2^-4 * A/448 * 2^-? absolute in the subnormal range) propagated through an orthogonal map
    amax = np.abs(ref).max(axis=(1, 2))
    err = np.abs(k_rot - ref).max(axis=(1, 2))
    assert np.all(err <= amax * 2 ** -4 * 1.5)
    # and the stored codes decode to the rotated keys within one more FP8 rounding
    _, k_hat, _ = dequant_ring(ring, head, filled)
    err2 = np.abs(k_hat - ref).max(axis=(1, 2))
    assert np.all(err2 <= amax * 2 ** -3 * 1.5)
    # values untouched
    assert np.array_equal(ring.v, before.v) and np.array_equal(ring.v_scale, before.v_scale)


def test_delta_then_minus_delta_is_identity_before_requantisation():
    ring, head, filled, _, _ = _steady_small()
    _, k_hat0, _ = dequant_ring(ring, head, filled)
    from oracle.rope import delta_cos_sin
    c, s = delta_cos_sin(777, ring.head_dim)
    c2, s2 = delta_cos_sin(-777, ring.head_dim)
    x = k_hat0.astype(np.float32)
    back = rope_rotate(rope_rotate(x, c, s), c2, s2)
    assert np.abs(back - x).max() <= 1e-6 * np.abs(x).max() * 4


def test_delta_zero_keeps_codes():
    # a ring holding one write: rotating by 0 re-derives the same scale (within 1 ulp) and
    # every code maps back to itself
    ring, head, filled, _, sched = _steady_small(writes=1)
    before = ring.copy()
    ring_delta_rotate(ring, head, filled, 0)
    assert np.array_equal(ring.k, before.k)
    vs = valid_slots(head, filled, ring.slots)
    a, b = ring.k_scale[:, vs], before.k_scale[:, vs]
    assert np.all(np.abs(a - b) <= np.spacing(b))
    # several writes: one new scale per head, equal (within 1 ulp) to the largest write scale,
    # and the codes of the write that held that maximum are unchanged
    ring, head, filled, _, sched = _steady_small(writes=3)
    before = ring.copy()
    ring_delta_rotate(ring, head, filled, 0)
    vs = valid_slots(head, filled, ring.slots)
    for h in range(ring.heads):
        bmax = before.k_scale[h, vs].max()
        assert np.all(np.abs(ring.k_scale[h, vs] - bmax) <= np.spacing(bmax))
        top = vs[before.k_scale[h, vs] == bmax]
        assert np.array_equal(ring.k[h, top], before.k[h, top])
    free = np.setdiff1d(np.arange(ring.slots), vs)
    assert np.array_equal(ring.k[:, free], before.k[:, free])


def _raw_valid(ring, head, filled, sched, name="dr"):
    """Raw (unquantised) keys/values of the valid slots and their positions, rebuilt from the seeds."""
    raw_k = np.zeros((ring.heads, ring.slots, ring.head_dim), np.float64)
    raw_v = np.zeros_like(raw_k)
    pos = np.zeros(ring.slots, np.int64)
    for w in sched:
        s = (w.start_slot + np.arange(w.n)) % ring.slots
        raw_k[:, s] = widen_bf16(_tokens(tensor_seed(name, w.pos0, 1), w.n, ring.heads, ring.head_dim)).transpose(1, 0, 2)
        raw_v[:, s] = widen_bf16(_tokens(tensor_seed(name, w.pos0, 2), w.n, ring.heads, ring.head_dim)).transpose(1, 0, 2)
        pos[s] = w.pos0 + np.arange(w.n)
    vs = valid_slots(head, filled, ring.slots)
    return raw_k[:, vs], raw_v[:, vs], pos[vs]


def _rot64(x, pos, d):
    freqs = 10000.0 ** (-np.arange(0, d, 2) / d)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None] * freqs[None, :])
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def test_delta_rotation_preserves_attention_when_queries_move_too():
    """Attention depends on relative positions only: after moving every key by delta and the
    queries by delta too, the oracle must be as close to the unquantised float64 attention at
    the original positions as it was before the move."""
    ring, head, filled, table, sched = _steady_small()
    d = ring.head_dim
    q = _tokens(99, 40, ring.heads, d)
    qp = sched[-1].pos0
    rk, rv, pos = _raw_valid(ring, head, filled, sched)
    qpos = qp + np.arange(40)
    exact = np.zeros((40, ring.heads, d))
    for h in range(ring.heads):
        qh = _rot64(widen_bf16(q)[:, h].astype(np.float64), qpos, d)
        kh = _rot64(rk[h], pos, d)
        exact[:, h], _ = softmax_attention(qh, kh, rv[h], 0.125)

    def rel(o):
        return (np.abs(o - exact).max(axis=(0, 2)) / np.abs(exact).max(axis=(0, 2))).max()

    out0, _ = ring_attention(ring, head, filled, q, qp, table, 0.125)
    moved = ring.copy()
    ring_delta_rotate(moved, head, filled, -250)
    out1, _ = ring_attention(moved, head, filled, q, qp - 250, table, 0.125)
    assert rel(out0) < 0.1
    assert rel(out1) < 2 * rel(out0) + 0.02
    # a rotation in the wrong direction is far off
    wrong = ring.copy()
    ring_delta_rotate(wrong, head, filled, +250)
    out2, _ = ring_attention(wrong, head, filled, q, qp - 250, table, 0.125)
    assert rel(out2) > 0.3


def test_query_quantisation_uses_one_scale_per_head():
    table = rope_table(64, 64)
    q = _tokens(3, 10, 3, 64)
    q_hat, codes, scale = q_prep(q, 7, table)
    assert codes.shape == (10, 3, 64) and scale.shape == (3,)
    # the largest rotated magnitude of each head maps to code 0x7E/0xFE (448)
    assert np.all((np.abs(codes.astype(np.int32) & 0x7F) == 0x7E).any(axis=(0, 2)))
    assert np.array_equal(np.abs(q_hat).max(axis=(0, 2)), 448.0 * scale.astype(np.float64))
