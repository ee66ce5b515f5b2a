"""Parity of the HIP library (through the C ABI) with the CPU oracle on the same seeded inputs.

Bars: ring codes and scales bit-exact (write and delta rotation); the FP8 encoder bit-exact
over every float32 in its rounding range; attention within 2e-2 infinity-norm relative error
per head (max |o - o_ref| / max |o_ref|) and 1e-3 absolute on the LSE."""

import math

import numpy as np
import pytest

import oracle
from workloads import (normal_bf16, student_t_outlier_bf16, outlier_channels, tensor_seed,
                       tiny_schedule, steady_ring_schedule, ROPE_POSITIONS, bf16_bits_from_f32,
                       f32_from_bf16_bits)

from kvhelpers import (ring_to_host, to_dev_bf16, bf16_dev_to_f64, attention_errors,
                       poison_free_slots_gpu, mfma_lse_bound)

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-2
LSE_TOL = 1e-3
# LSE bar of the position-reset workload (Student-t keys with x20 outlier channels): the FP8
# matrix core's grouped accumulation truncates small products next to outlier products, which
# moves scores by up to a few hundredths; measured maximum 4.7e-2 over all 24 x 757 entries.
OUTLIER_LSE_TOL = 6e-2


@pytest.fixture(scope="module")
def torch():
    import torch
    return torch


@pytest.fixture(scope="module")
def kv():
    import fp8_ring_kv_write_amd as kv
    return kv


_TABLES = {}


def tables(kv, torch, d, n_pos=ROPE_POSITIONS):
    key = (d, n_pos)
    if key not in _TABLES:
        host = kv.rope_table(n_pos, d)
        ref = oracle.rope_table(n_pos, d)
        assert host.tobytes() == ref.tobytes()
        _TABLES[key] = (torch.from_numpy(host).cuda(), ref)
    return _TABLES[key]


class Pair:
    """The same ring in the library (GPU) and in the oracle (CPU)."""

    def __init__(self, kv, torch, heads, slots, d):
        self.kv, self.torch = kv, torch
        self.g = kv.Ring(heads, slots, d)
        self.o = oracle.OracleRing(heads, slots, d)
        self.head, self.filled = 0, 0
        self.tab_dev, self.tab = tables(kv, torch, d)

    def write(self, k_bits, v_bits, start, pos0):
        self.kv.kv_ring_write(self.g, to_dev_bf16(k_bits), to_dev_bf16(v_bits), start, pos0, self.tab_dev)
        oracle.ring_write(self.o, k_bits, v_bits, start, pos0, self.tab)
        self.head, self.filled = oracle.advance(start, k_bits.shape[0], self.filled, self.o.slots)

    def assert_same(self, what=""):
        self.torch.cuda.synchronize()
        k, v, ks, vs = ring_to_host(self.g)
        assert np.array_equal(k, self.o.k), f"K codes differ {what}: {np.argwhere(k != self.o.k)[:5]}"
        assert np.array_equal(v, self.o.v), f"V codes differ {what}: {np.argwhere(v != self.o.v)[:5]}"
        assert np.array_equal(ks, self.o.k_scale), f"K scales differ {what}"
        assert np.array_equal(vs, self.o.v_scale), f"V scales differ {what}"

    def attend(self, q_bits, q_pos0, scale, heads=None):
        out, lse = self.kv.ring_attention(self.g, self.head, self.filled, to_dev_bf16(q_bits), q_pos0,
                                          self.tab_dev, scale)
        self.torch.cuda.synchronize()
        ref_o, ref_l = oracle.ring_attention(self.o, self.head, self.filled, q_bits, q_pos0, self.tab,
                                             scale, heads=heads)
        return bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ref_o, ref_l


def check_attention(out, lse, ref_o, ref_l, heads=None, tol=ATT_TOL, label="", lse_tol=LSE_TOL):
    """Output within `tol` (per-head infinity-norm relative error); every LSE entry within
    `lse_tol` (absolute)."""
    hs = list(range(out.shape[1])) if heads is None else heads
    inf_rel, l2_rel = attention_errors(out[:, hs], ref_o[:, hs])
    lse_dev = np.abs(lse[hs] - ref_l[hs])
    print(f"[{label}] inf-rel max {inf_rel.max():.2e} (mean {inf_rel.mean():.2e}), "
          f"L2-rel max {l2_rel.max():.2e}, lse abs max {lse_dev.max():.2e}", flush=True)
    assert np.all(np.isfinite(out[:, hs]))
    assert inf_rel.max() <= tol, inf_rel
    assert np.all(np.isfinite(lse[hs]) == np.isfinite(ref_l[hs]))
    assert lse_dev[np.isfinite(lse_dev)].max(initial=0.0) <= lse_tol, lse_dev.max()


# ------------------------------------------------------------------ FP8 encoder

def _encoder_sweep(kv, torch, sign):
    """Every float32 of the given sign with magnitude in [2^-12, 2^10): all of E4M3's rounding
    decisions (subnormals, every binade, saturation above 448), against the oracle."""
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** 10).view(np.uint32)
    step = 1 << 24
    for start in range(int(lo), int(hi), step):
        bits = np.arange(start, min(start + step, int(hi)), dtype=np.uint32)
        if sign < 0:
            bits |= np.uint32(0x80000000)
        x = bits.view(np.float32)
        got = kv.fp8_encode(torch.from_numpy(x).cuda()).cpu().numpy()
        ref = oracle.e4m3_encode(x)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_fp8_encoder_exhaustive_positive(kv, torch):
    """Positive inputs, exhaustively over the rounding range; below 2^-12 and above 2^10 (both
    signs) on a stride."""
    _encoder_sweep(kv, torch, +1)
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** 10).view(np.uint32)
    rest = np.concatenate([
        np.arange(0, int(lo), 997, dtype=np.uint32),
        np.arange(int(hi), 0x7F800000, 997, dtype=np.uint32),
    ]).view(np.float32)
    for x in (rest, -rest):
        x = np.ascontiguousarray(x)
        got = kv.fp8_encode(torch.from_numpy(x).cuda()).cpu().numpy()
        assert np.array_equal(got, oracle.e4m3_encode(x))


def test_fp8_encoder_exhaustive_negative(kv, torch):
    """Negative inputs, exhaustively over the rounding range."""
    _encoder_sweep(kv, torch, -1)


# ------------------------------------------------------------------ write

def test_tiny_schedule_write_and_attention(kv, torch):
    """The tiny workload: 1 head, d64, 64 slots, six writes of 16 (the ring fills, then wraps);
    codes bit-exact after every write, attention of the 16 new queries over the filled slots."""
    p = Pair(kv, torch, 1, 64, 64)
    for wi, w in enumerate(tiny_schedule()):
        k = normal_bf16(tensor_seed("tiny", wi, 1), (16, 1, 64))
        v = normal_bf16(tensor_seed("tiny", wi, 2), (16, 1, 64))
        q = normal_bf16(tensor_seed("tiny", wi, 0), (16, 1, 64))
        p.write(k, v, w.start_slot, w.pos0)
        p.assert_same(f"after write {wi}")
        check_attention(*p.attend(q, w.pos0, 1 / 8), label=f"tiny write {wi} filled {p.filled}")


def test_write_path_full_size_wraps(kv, torch):
    """757 tokens x 24 heads x d128 into a 5,788-slot ring starting at slot 5,500 (288 slots,
    then 469 after the wrap), positions 12,000.., then a second write right after it."""
    p = Pair(kv, torch, 24, 5788, 128)
    k = normal_bf16(tensor_seed("write_path", 0, 1), (757, 24, 128))
    v = normal_bf16(tensor_seed("write_path", 0, 2), (757, 24, 128))
    p.write(k, v, 5500, 12000)
    p.assert_same("first write")
    k2 = normal_bf16(tensor_seed("write_path", 1, 1), (757, 24, 128))
    v2 = normal_bf16(tensor_seed("write_path", 1, 2), (757, 24, 128))
    p.write(k2, v2, p.head, 12757)
    p.assert_same("second write")


def test_write_whole_ring_more_work_groups_than_fit(kv, torch):
    """A write of the whole 5,788-slot ring, 24 heads x d128, from slot 3,001 (it wraps; 181
    chunks per head): 4,344 work-groups, more than the GPU holds at once, so every per-head
    wait relies on each XCD starting its heads in order.  Bytes bit-exact, no wait at its
    bound."""
    p = Pair(kv, torch, 24, 5788, 128)
    k = normal_bf16(tensor_seed("whole_ring", 0, 1), (5788, 24, 128))
    v = normal_bf16(tensor_seed("whole_ring", 0, 2), (5788, 24, 128))
    p.write(k, v, 3001, 4000)
    p.assert_same("whole-ring write")
    assert kv.sync_status() == 0


@pytest.mark.parametrize("heads,slots,d,writes", [
    (3, 203, 128, [(1, 0, 0), (203, 5, 1), (7, 200, 300), (64, 101, 400), (130, 150, 600)]),
    (2, 64, 64, [(64, 0, 0), (1, 63, 64), (33, 17, 100)]),
    (1, 1, 128, [(1, 0, 3), (1, 0, 4)]),
])
def test_write_edge_shapes(kv, torch, heads, slots, d, writes):
    """Ragged rings (slots not a multiple of 4, 32 or 128), writes of 1 token, of the whole
    ring, and wrapping writes that meet their own start in one chunk."""
    p = Pair(kv, torch, heads, slots, d)
    for j, (n, start, pos0) in enumerate(writes):
        k = normal_bf16(tensor_seed("edge", slots, j, 1), (n, heads, d))
        v = normal_bf16(tensor_seed("edge", slots, j, 2), (n, heads, d))
        p.write(k, v, start, pos0)
        p.assert_same(f"write {j}")


def test_write_zero_and_outlier_heads(kv, torch):
    """A head of zeros (absmax floor), Student-t values with outlier channels."""
    p = Pair(kv, torch, 4, 300, 128)
    out = outlier_channels(tensor_seed("zo", 9), 4, 128)
    k = student_t_outlier_bf16(tensor_seed("zo", 1), (100, 4, 128), out)
    v = student_t_outlier_bf16(tensor_seed("zo", 2), (100, 4, 128), out)
    k[:, 1, :] = 0
    v[:, 2, :] = 0x8000   # negative zeros
    p.write(k, v, 250, 77)
    p.assert_same("zero/outlier heads")


# ------------------------------------------------------------------ delta rotation

def _fill_steady(p, name, n, writes, pos_offset=0, dist="normal", outliers=None):
    H, S, D = p.o.heads, p.o.slots, p.o.head_dim
    for c, w in enumerate(steady_ring_schedule(S, n, writes, pos_offset)):
        if dist == "normal":
            k = normal_bf16(tensor_seed(name, c, 1), (n, H, D))
            v = normal_bf16(tensor_seed(name, c, 2), (n, H, D))
        else:
            k = student_t_outlier_bf16(tensor_seed(name, c, 1), (n, H, D), outliers)
            v = student_t_outlier_bf16(tensor_seed(name, c, 2), (n, H, D), outliers)
        p.write(k, v, w.start_slot, w.pos0)
    return steady_ring_schedule(S, n, writes, pos_offset)


@pytest.mark.parametrize("slots,n,writes,delta,base", [
    (203, 48, 3, -100, 10000.0),     # partially filled ring
    (203, 48, 7, 37, 10000.0),       # full, wrapped
    (203, 48, 2, 0, 10000.0),        # delta 0
    (203, 48, 7, -1234, 500000.0),   # another rotary base
    (203, 48, 7, (1 << 31) - 1, 10000.0),   # the largest delta (angles of about 2^31 radians)
])
def test_delta_rotate_small(kv, torch, slots, n, writes, delta, base):
    p = Pair(kv, torch, 3, slots, 128)
    _fill_steady(p, f"drs{slots}{writes}", n, writes, pos_offset=500)
    p.assert_same("before rotation")
    kv.kv_ring_delta_rotate(p.g, p.head, p.filled, delta, rope_base=base)
    oracle.ring_delta_rotate(p.o, p.head, p.filled, delta, base=base)
    p.assert_same(f"after delta {delta} (base {base})")


def test_reset_outliers_one_layer_full_size(kv, torch):
    """One layer of the reset workload: 24 heads x d128 x 5,788 slots filled with Student-t(3)
    keys/values whose 1% outlier channels are x20, positions 6,212..11,999; delta = -4,000;
    then 757 queries at 7,243..7,999."""
    p = Pair(kv, torch, 24, 5788, 128)
    outl = outlier_channels(tensor_seed("reset", 0, 3), 24, 128)
    sched = _fill_steady(p, "reset_l0", 757, 8, pos_offset=5944, dist="t", outliers=outl)
    p.assert_same("filled")
    kv.kv_ring_delta_rotate(p.g, p.head, p.filled, -4000)
    oracle.ring_delta_rotate(p.o, p.head, p.filled, -4000)
    p.assert_same("after delta -4000")
    q = normal_bf16(tensor_seed("reset_l0", 99, 0), (757, 24, 128))
    qp = sched[-1].pos0 - 4000
    out, lse, ro, rl = p.attend(q, qp, 1 / math.sqrt(128))
    # LSE: every one of the 24 x 757 entries against OUTLIER_LSE_TOL.  The outlier channels make
    # products inside one 8-channel group of the FP8 matrix core differ by more than 2^13, where
    # its grouped accumulation truncates the small ones; the derived per-query bound of that
    # truncation is printed beside the measured deviation on 12 queries per head (diagnostic).
    check_attention(out, lse, ro, rl, label="reset outliers", lse_tol=OUTLIER_LSE_TOL)
    q_hat, _, _ = oracle.q_prep(q, qp, p.tab)
    _, k_hat, _ = oracle.kvcache.dequant_ring(p.o, p.head, p.filled)
    sample = np.linspace(0, 756, 12).astype(int)
    ratio = max((np.abs(lse[h, sample] - rl[h, sample]) /
                 (LSE_TOL + mfma_lse_bound(q_hat[sample, h, :], k_hat[h], 1 / math.sqrt(128)))).max()
                for h in range(24))
    print(f"[reset outliers] lse deviation / (1e-3 + grouped-accumulation bound), max over "
          f"12 x 24 sampled entries: {ratio:.2f}", flush=True)


# ------------------------------------------------------------------ attention

def test_attention_single_call_full_size(kv, torch):
    """757 queries against a full 5,788-slot ring, 24 heads x d128 (the ring built by 8 writes of
    757; the last one wraps)."""
    p = Pair(kv, torch, 24, 5788, 128)
    sched = _fill_steady(p, "single_call", 757, 8)
    assert (p.head, p.filled) == (268, 5788)
    p.assert_same("steady ring")
    q = normal_bf16(tensor_seed("single_call", 99, 0), (757, 24, 128))
    out, lse, ro, rl = p.attend(q, sched[-1].pos0, 1 / math.sqrt(128))
    check_attention(out, lse, ro, rl, label="single call")


def test_attention_fill_up_full_size(kv, torch):
    """The first chunks of a session: 757 queries over a 24-head d128 ring of 5,788 slots that
    holds one, two and then three 757-token chunks (rows of 6, 12 and 18 tiles: one work-group
    per row for the first two, rows split between work-groups for the third)."""
    p = Pair(kv, torch, 24, 5788, 128)
    for c in range(3):
        k = normal_bf16(tensor_seed("fill_up", c, 1), (757, 24, 128))
        v = normal_bf16(tensor_seed("fill_up", c, 2), (757, 24, 128))
        p.write(k, v, 757 * c, 757 * c)
        assert (p.head, p.filled) == (757 * (c + 1), 757 * (c + 1))
        q = normal_bf16(tensor_seed("fill_up", c, 0), (757, 24, 128))
        check_attention(*p.attend(q, 757 * c, 1 / math.sqrt(128)), label=f"fill-up filled={p.filled}")
    p.assert_same("after three chunks")


@pytest.mark.parametrize("slots,n,writes,nq", [
    (700, 100, 3, 1),       # partial ring, one query
    (700, 100, 8, 17),      # wrapped full ring, ragged queries
    (700, 100, 5, 129),     # partial, queries over two tiles of 128
    (64, 16, 2, 16),
])
def test_attention_partial_and_ragged(kv, torch, slots, n, writes, nq):
    p = Pair(kv, torch, 2, slots, 128)
    sched = _fill_steady(p, f"pr{slots}{writes}{nq}", n, writes)
    q = normal_bf16(tensor_seed("prq", slots, writes, nq), (nq, 2, 128))
    check_attention(*p.attend(q, sched[-1].pos0, 1 / math.sqrt(128)),
                    label=f"S={slots} filled={p.filled} nq={nq}")


@pytest.mark.parametrize("scale", [1e-3, 2.0, 8.0])
def test_attention_softmax_scale_extremes(kv, torch, scale):
    """Softmax scales far from 1/sqrt(d): nearly uniform weights (1e-3) and sharp ones (2 and 8,
    where a few slots carry almost all the weight and the running max moves by far more than
    the lazy rescale's threshold), over a wrapped 700-slot ring, 3 heads x d128, 129 queries."""
    p = Pair(kv, torch, 3, 700, 128)
    sched = _fill_steady(p, "scale_extremes", 100, 8)
    q = normal_bf16(tensor_seed("scale_extremes", 9, 0), (129, 3, 128))
    # The LSE is in units of scaled scores: the bar holds the error of the unscaled score q.k to
    # what 1e-3 allows at the standard scale 1/sqrt(d), i.e. 1e-3 * scale * sqrt(d) above it.
    lse_tol = LSE_TOL * max(1.0, scale * math.sqrt(128))
    check_attention(*p.attend(q, sched[-1].pos0, scale), label=f"softmax scale {scale}", lse_tol=lse_tol)


def test_attention_ignores_poisoned_free_slots(kv, torch):
    p = Pair(kv, torch, 2, 700, 128)
    sched = _fill_steady(p, "poison", 100, 4)     # 400 of 700 slots
    q = normal_bf16(tensor_seed("poison", 9, 0), (130, 2, 128))
    out0, lse0, ro, rl = p.attend(q, sched[-1].pos0, 1 / math.sqrt(128))
    poison_free_slots_gpu(p.g, oracle.valid_slots(p.head, p.filled, 700))
    out1, lse1, _, _ = p.attend(q, sched[-1].pos0, 1 / math.sqrt(128))
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    check_attention(out1, lse1, ro, rl, label="poisoned")


@pytest.mark.parametrize("d", [128, 64])
def test_attention_mixed_write_scales(kv, torch, d):
    """A ring whose writes differ in scale by orders of magnitude, with write boundaries inside
    tiles: N(0,1) writes, an all-zero write (its scales at the absmax floor, 2^-100 / 448), a
    write with K x4 and V x1000 and one with V x1e-3.  The attention forms its probabilities
    against the running max of score plus log2 of the slot's V scale, so slots of very
    different V scales meet in one tile and across tiles."""
    H, S, n = 3, 700, 100
    p = Pair(kv, torch, H, S, d)
    sched = steady_ring_schedule(S, n, 8)          # 800 tokens: the last write wraps
    for c, w in enumerate(sched):
        k = normal_bf16(tensor_seed("mixed_scales", d, c, 1), (n, H, d))
        v = normal_bf16(tensor_seed("mixed_scales", d, c, 2), (n, H, d))
        if c == 2:
            k[:] = 0
            v[:] = 0
        elif c == 4:
            k = bf16_bits_from_f32(f32_from_bf16_bits(k) * np.float32(4.0))
            v = bf16_bits_from_f32(f32_from_bf16_bits(v) * np.float32(1000.0))
        elif c == 6:
            v = bf16_bits_from_f32(f32_from_bf16_bits(v) * np.float32(1e-3))
        p.write(k, v, w.start_slot, w.pos0)
    p.assert_same("mixed write scales")
    q = normal_bf16(tensor_seed("mixed_scales", d, 99, 0), (150, H, d))
    check_attention(*p.attend(q, sched[-1].pos0, 1 / math.sqrt(d)), label=f"mixed write scales d{d}")


def test_large_ring_long_writes_and_rotation(kv, torch):
    """A ring of 20,000 slots (157 tiles per head) filled by writes of 5,000 tokens (the last one
    wraps): the write's partial-max lists (157 groups per head) and the delta rotation's (157
    tiles) are longer than a wavefront and take the work-group reduction; ring bytes bit-exact
    after the writes and after a rotation, attention over the whole ring before and after it."""
    H, S, D, n = 2, 20000, 128, 5000
    p = Pair(kv, torch, H, S, D)
    for c in range(5):                     # slots 0, 5,000, ..., 20,000 -> 0: the fifth wraps
        k = normal_bf16(tensor_seed("large_ring", c, 1), (n, H, D))
        v = normal_bf16(tensor_seed("large_ring", c, 2), (n, H, D))
        p.write(k, v, (n * c) % S, 2000 * c)   # positions 0 .. 12,999, inside the rotary table
    assert (p.head, p.filled) == (5000, S)
    p.assert_same("large ring")
    q = normal_bf16(tensor_seed("large_ring", 9, 0), (200, H, D))
    check_attention(*p.attend(q, 9000, 1 / math.sqrt(D)), label="large ring")
    kv.kv_ring_delta_rotate(p.g, p.head, p.filled, -3000)
    oracle.ring_delta_rotate(p.o, p.head, p.filled, -3000)
    p.assert_same("large ring after delta -3000")
    check_attention(*p.attend(q, 6000, 1 / math.sqrt(D)), label="large ring after rotation")


def test_largest_head_count(kv, torch):
    """512 heads (the most the synchronisation records hold) x 300 slots x d64: every head's record
    in use, writes of 3,584 and 3,072 work-groups taken in the write's XCD order, a rotation, and
    an attention whose 512 rows outnumber the work-groups.  Bytes bit-exact, attention within the bar, no wait at
    its bound."""
    H, S, D = 512, 300, 64
    p = Pair(kv, torch, H, S, D)
    for c, (n, start, pos0) in enumerate([(200, 0, 0), (150, 200, 500)]):   # the second wraps
        k = normal_bf16(tensor_seed("max_heads", c, 1), (n, H, D))
        v = normal_bf16(tensor_seed("max_heads", c, 2), (n, H, D))
        p.write(k, v, start, pos0)
    assert (p.head, p.filled) == (50, 300)
    p.assert_same("512 heads")
    kv.kv_ring_delta_rotate(p.g, p.head, p.filled, -50)
    oracle.ring_delta_rotate(p.o, p.head, p.filled, -50)
    p.assert_same("512 heads after delta -50")
    q = normal_bf16(tensor_seed("max_heads", 9, 0), (17, H, D))
    check_attention(*p.attend(q, 600, 1 / math.sqrt(D)), label="512 heads")
    assert kv.sync_status() == 0


def test_largest_slot_count(kv, torch):
    """A ring of 2^20 slots (the most a ring may have; 8,192 tiles per head), 2 heads x d128,
    written near its end so that the last write wraps to slot 0: slot and byte offsets at the
    top of their range, a rotation and an attention over the wrapped valid interval."""
    H, S, D, n = 2, 1 << 20, 128, 4000
    p = Pair(kv, torch, H, S, D)
    start = S - 6000
    for c in range(3):                     # slots S-6000 .. S-1, then 0 .. 5,999
        k = normal_bf16(tensor_seed("max_slots", c, 1), (n, H, D))
        v = normal_bf16(tensor_seed("max_slots", c, 2), (n, H, D))
        p.write(k, v, (start + n * c) % S, n * c)
    assert (p.head, p.filled) == (6000, 12000)
    p.assert_same("2^20 slots")
    kv.kv_ring_delta_rotate(p.g, p.head, p.filled, -700)
    oracle.ring_delta_rotate(p.o, p.head, p.filled, -700)
    p.assert_same("2^20 slots after delta -700")
    q = normal_bf16(tensor_seed("max_slots", 9, 0), (5, H, D))
    check_attention(*p.attend(q, 11000, 1 / math.sqrt(D)), label="2^20 slots")
    assert kv.sync_status() == 0


def test_write_and_attention_at_the_token_limit(kv, torch):
    """One write of KV_RING_MAX_TOKENS = 16,384 tokens (8 heads x d64 into a 20,000-slot ring,
    wrapping): 513 work-groups per head, about 65 on each XCD, 4,104 in all, more than the GPU
    holds at once; then an attention of 16,384 queries (64 rows per head), checked on two heads."""
    H, S, D, n = 8, 20000, 64, kv.MAX_TOKENS
    p = Pair(kv, torch, H, S, D)
    k = normal_bf16(tensor_seed("token_limit", 0, 1), (n, H, D))
    v = normal_bf16(tensor_seed("token_limit", 0, 2), (n, H, D))
    p.write(k, v, 10000, 0)
    assert (p.head, p.filled) == ((10000 + n) % S, n)
    p.assert_same("16,384-token write")
    q = normal_bf16(tensor_seed("token_limit", 9, 0), (n, H, D))
    check_attention(*p.attend(q, 0, 1 / math.sqrt(D), heads=[0, 5]), heads=[0, 5], label="16,384 queries")
    assert kv.sync_status() == 0


def test_attention_empty_ring_and_no_queries(kv, torch):
    g = kv.Ring(2, 300, 128)
    tab_dev, _ = tables(kv, torch, 128)
    q = to_dev_bf16(normal_bf16(1, (20, 2, 128)))
    out, lse = kv.ring_attention(g, 0, 0, q, 0, tab_dev, 0.1)
    torch.cuda.synchronize()
    assert np.all(bf16_dev_to_f64(out) == 0)
    assert np.all(np.isneginf(lse.cpu().numpy()))
    kv.ring_attention(g, 0, 10, q[:0], 0, tab_dev, 0.1)   # nq = 0: nothing happens


def test_attention_is_deterministic(kv, torch):
    p = Pair(kv, torch, 4, 1000, 128)
    sched = _fill_steady(p, "det", 300, 4)
    q = to_dev_bf16(normal_bf16(5, (300, 4, 128)))
    o1, l1 = kv.ring_attention(p.g, p.head, p.filled, q, sched[-1].pos0, p.tab_dev, 0.09)
    o2, l2 = kv.ring_attention(p.g, p.head, p.filled, q, sched[-1].pos0, p.tab_dev, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ------------------------------------------------------------------ read-time baseline

@pytest.mark.parametrize("w,n,row", [(5788, 757, (24, 128)), (300, 0, (2, 64)), (300, 300, (2, 64)),
                                     (97, 1, (8,)), (97, 96, (3, 40))])
def test_window_advance_bit_exact(kv, torch, w, n, row):
    rng = np.random.default_rng(w + n)
    win = rng.integers(0, 1 << 16, size=(w, *row), dtype=np.uint16)
    fresh = rng.integers(0, 1 << 16, size=(n, *row), dtype=np.uint16)
    src, fr = to_dev_bf16(win), to_dev_bf16(fresh)
    dst = torch.full_like(src, float("nan"))
    kv.kv_window_advance(src, dst, fr)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.window_advance(win, fresh))
    if n < w:   # the copy never writes over what it reads
        with pytest.raises(kv.KvRingError):
            kv.kv_window_advance(src, src, fr)


def test_read_time_call_full_size(kv, torch):
    """The read-time design on one layer: a 5,788-token bfloat16 window (positions 6,212 ..
    11,999 after the advance) moves forward by 757 tokens, the whole window is rotated and
    quantised again (one write of 5,788 tokens into a ring of 5,788 slots at slot 0), then 757
    queries at the newest positions attend over it."""
    w, n, h, d, p_new = 5788, 757, 24, 128, 6212
    old_k = normal_bf16(tensor_seed("read_time", 0, 1), (w, h, d))
    old_v = normal_bf16(tensor_seed("read_time", 0, 2), (w, h, d))
    new_k = normal_bf16(tensor_seed("read_time", 1, 1), (n, h, d))
    new_v = normal_bf16(tensor_seed("read_time", 1, 2), (n, h, d))
    q = normal_bf16(tensor_seed("read_time", 1, 0), (n, h, d))
    wk, wv = oracle.window_advance(old_k, new_k), oracle.window_advance(old_v, new_v)
    dk, dv = torch.empty((w, h, d), dtype=torch.bfloat16, device="cuda"), torch.empty(
        (w, h, d), dtype=torch.bfloat16, device="cuda")
    kv.kv_window_advance(to_dev_bf16(old_k), dk, to_dev_bf16(new_k))
    kv.kv_window_advance(to_dev_bf16(old_v), dv, to_dev_bf16(new_v))
    p = Pair(kv, torch, h, w, d)
    kv.kv_ring_write(p.g, dk, dv, 0, p_new, p.tab_dev)
    p.o = oracle.read_time_ring(wk, wv, p_new, p.tab)
    p.head, p.filled = 0, w
    p.assert_same("read-time window")
    out, lse, ro, rl = p.attend(q, p_new + w - n, 1 / math.sqrt(d))
    check_attention(out, lse, ro, rl, label="read-time call")


# ------------------------------------------------------------------ graph capture

def test_layer_calls_replay_from_a_captured_graph(kv, torch):
    """Write + attention on two rings captured once in a HIP graph (no call allocates, memsets or
    synchronises), replayed three times with eager work and synchronisation in between: every
    replay leaves exactly the rings, outputs and LSE that the same calls leave when run eagerly."""
    h, s, d, n = 4, 700, 128, 100
    tab_dev, _ = tables(kv, torch, d)
    rings = [kv.Ring(h, s, d), kv.Ring(h, s, d)]
    for r in rings:
        for c in range(6):
            kv.kv_ring_write(r, to_dev_bf16(normal_bf16(tensor_seed("graph", c, 1), (n, h, d))),
                             to_dev_bf16(normal_bf16(tensor_seed("graph", c, 2), (n, h, d))),
                             (c * n) % s, c * n, tab_dev)
    head, filled = (6 * n) % s, 6 * n
    k_new = [to_dev_bf16(normal_bf16(tensor_seed("graph", 10 + i, 1), (n, h, d))) for i in range(2)]
    v_new = [to_dev_bf16(normal_bf16(tensor_seed("graph", 10 + i, 2), (n, h, d))) for i in range(2)]
    q = [to_dev_bf16(normal_bf16(tensor_seed("graph", 10 + i, 0), (n, h, d))) for i in range(2)]
    ws_w = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, h, s, d, n), dtype=torch.uint8, device="cuda")
    ws_a = torch.zeros(kv.workspace_bytes(kv.OP_ATTENTION, h, s, d, n), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q[0]) for _ in range(2)]
    lses = [torch.empty((h, n), dtype=torch.float32, device="cuda") for _ in range(2)]
    start, pos0 = (head - n) % s, 5 * n
    snap = [(r.k.clone(), r.v.clone(), r.k_scale.clone(), r.v_scale.clone()) for r in rings]

    def calls():
        for i, r in enumerate(rings):
            kv.kv_ring_write(r, k_new[i], v_new[i], start, pos0, tab_dev, workspace=ws_w)
            kv.ring_attention(r, head, filled, q[i], pos0, tab_dev, 0.09, out=outs[i], lse=lses[i],
                              workspace=ws_a)

    def restore():
        for r, (k, v, ks, vs) in zip(rings, snap):
            r.k.copy_(k), r.v.copy_(v), r.k_scale.copy_(ks), r.v_scale.copy_(vs)

    def state():
        return [t.clone() for r in rings for t in (r.k, r.v, r.k_scale, r.v_scale)] + \
               [t.clone() for t in outs + lses]

    calls()
    torch.cuda.synchronize()
    eager = state()
    restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm the side stream before capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        for t in outs + lses:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        for a, b in zip(got, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        _ = (q[0].float() * 2).sum().item()   # eager work between replays


# ------------------------------------------------------------------ fused layer call

@pytest.mark.parametrize("heads,slots,d,n,nq,writes", [
    (24, 5788, 128, 757, 757, 8),    # the steady-state layer call (the last write wraps)
    (2, 100, 128, 77, 77, 3),        # queries = new tokens (prepared by the write's work-groups):
    (3, 64, 128, 1, 1, 3),           #   a write that wraps, one token, one whole 256-query row
    (2, 600, 128, 256, 256, 2),
    (3, 700, 128, 16, 129, 5),       # more queries than new tokens
    (2, 300, 64, 100, 1, 4),
    (2, 300, 128, 77, 0, 2),         # no queries: the write alone
    (8, 20000, 128, 16384, 16384, 1),  # the token limit, the queries prepared by the write's work-groups
])
def test_write_attend_equals_write_then_attention(kv, torch, heads, slots, d, n, nq, writes):
    """kv_ring_write_attend leaves the same ring bytes, outputs and LSE, bit for bit, as
    kv_ring_write followed by ring_attention."""
    tab_dev, _ = tables(kv, torch, d)
    rings = [kv.Ring(heads, slots, d), kv.Ring(heads, slots, d)]
    filled = 0
    for c in range(writes - 1):
        kk = to_dev_bf16(normal_bf16(tensor_seed("fused", c, 1), (n, heads, d)))
        vv = to_dev_bf16(normal_bf16(tensor_seed("fused", c, 2), (n, heads, d)))
        for r in rings:
            kv.kv_ring_write(r, kk, vv, (c * n) % slots, c * n, tab_dev)
        filled = min(filled + n, slots)
    c = writes - 1
    start, pos0 = (c * n) % slots, c * n
    head, filled = oracle.advance(start, n, filled, slots)
    kk = to_dev_bf16(normal_bf16(tensor_seed("fused", c, 1), (n, heads, d)))
    vv = to_dev_bf16(normal_bf16(tensor_seed("fused", c, 2), (n, heads, d)))
    q = to_dev_bf16(normal_bf16(tensor_seed("fused", c, 0), (nq, heads, d)))
    q_pos0 = pos0 + n - nq if nq <= pos0 + n else 0
    kv.kv_ring_write(rings[0], kk, vv, start, pos0, tab_dev)
    o1, l1 = kv.ring_attention(rings[0], head, filled, q, q_pos0, tab_dev, 1 / math.sqrt(d))
    o2, l2 = kv.kv_ring_write_attend(rings[1], kk, vv, start, pos0, head, filled, q, q_pos0, tab_dev,
                                     1 / math.sqrt(d))
    torch.cuda.synchronize()
    for a, b in ((rings[0].k, rings[1].k), (rings[0].v, rings[1].v),
                 (rings[0].k_scale, rings[1].k_scale), (rings[0].v_scale, rings[1].v_scale)):
        assert torch.equal(a, b)
    if nq:
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# ------------------------------------------------------------------ more shapes

def test_single_slot_ring(kv, torch):
    """A ring of one slot: every write replaces it, the attention has one valid key."""
    p = Pair(kv, torch, 2, 1, 128)
    for c in range(3):
        p.write(normal_bf16(tensor_seed("one_slot", c, 1), (1, 2, 128)),
                normal_bf16(tensor_seed("one_slot", c, 2), (1, 2, 128)), 0, c)
        p.assert_same(f"write {c}")
    assert (p.head, p.filled) == (0, 1)
    q = normal_bf16(tensor_seed("one_slot", 9, 0), (3, 2, 128))
    check_attention(*p.attend(q, 0, 1 / math.sqrt(128)), label="one slot")


def test_attention_head_dim_64_full_size(kv, torch):
    """The steady-state call with head_dim 64: 757 queries over a full 5,788-slot ring, 24 heads."""
    p = Pair(kv, torch, 24, 5788, 64)
    sched = _fill_steady(p, "d64_full", 757, 8)
    p.assert_same("steady ring d64")
    q = normal_bf16(tensor_seed("d64_full", 99, 0), (757, 24, 64))
    check_attention(*p.attend(q, sched[-1].pos0, 1 / math.sqrt(64)), label="d64 single call")


def test_attention_more_rows_than_work_groups(kv, torch):
    """1,500 queries x 24 heads = 288 rows of 128 queries, more rows than the 256 work-groups of
    the persistent grid, over a partly filled ring that wraps."""
    p = Pair(kv, torch, 24, 700, 128)
    sched = _fill_steady(p, "many_rows", 150, 6)     # 900 tokens: wraps, ring full
    q = normal_bf16(tensor_seed("many_rows", 9, 0), (1500, 24, 128))
    check_attention(*p.attend(q, 0, 1 / math.sqrt(128)), label="288 rows")


def test_attention_many_segments_per_work_group(kv, torch):
    """2,000 queries x 24 heads over a 2,000-slot ring: 384 rows of 16 tiles, so most work-groups
    run two or three segments (rows) one after the other."""
    p = Pair(kv, torch, 24, 2000, 128)
    sched = _fill_steady(p, "many_segs", 500, 5)     # 2,500 tokens: wraps, ring full
    q = normal_bf16(tensor_seed("many_segs", 9, 0), (2000, 24, 128))
    check_attention(*p.attend(q, 500, 1 / math.sqrt(128)), label="384 rows of 16 tiles")


def test_attention_rows_split_seven_ways(kv, torch):
    """One head, 300 queries over a full 5,788-slot ring: 2 rows of 46 tiles over a grid of 13
    work-groups (no XCD renumbering: 13 is not a multiple of 8), so every row is split between
    7 work-groups and its merge reads its segments in two batches."""
    p = Pair(kv, torch, 1, 5788, 128)
    _fill_steady(p, "seven_ways", 757, 8)             # 6,056 tokens: wraps, ring full
    q = normal_bf16(tensor_seed("seven_ways", 9, 0), (300, 1, 128))
    check_attention(*p.attend(q, 6000, 1 / math.sqrt(128)), label="rows split 7 ways")


def test_chunk_passes_rewrite_the_same_slots(kv, torch):
    """A chunk of the method on two layers: each of four denoising passes rewrites the chunk's
    slots at the same positions and attends (through kv_ring_write_attend); the ring head moves
    after the last pass.  Every pass's ring bytes and attention are checked against the oracle."""
    h, s, d, n = 4, 700, 128, 100
    tab_dev, tab = tables(kv, torch, d)
    for layer in range(2):
        p = Pair(kv, torch, h, s, d)
        sched = _fill_steady(p, f"chunk{layer}", n, 6)      # 600 of 700 slots, head 600
        start, pos0 = p.head, sched[-1].pos0 + n             # the new chunk's slots and positions
        head, filled = oracle.advance(start, n, p.filled, s)
        for ps in range(4):
            k = normal_bf16(tensor_seed("chunkpass", layer, ps, 1), (n, h, d))
            v = normal_bf16(tensor_seed("chunkpass", layer, ps, 2), (n, h, d))
            q = normal_bf16(tensor_seed("chunkpass", layer, ps, 0), (n, h, d))
            out, lse = kv.kv_ring_write_attend(p.g, to_dev_bf16(k), to_dev_bf16(v), start, pos0, head,
                                               filled, to_dev_bf16(q), pos0, tab_dev, 1 / math.sqrt(d))
            torch.cuda.synchronize()
            oracle.ring_write(p.o, k, v, start, pos0, tab)
            p.head, p.filled = head, filled
            p.assert_same(f"layer {layer} pass {ps}")
            ro, rl = oracle.ring_attention(p.o, head, filled, q, pos0, tab, 1 / math.sqrt(d))
            check_attention(bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl,
                            label=f"layer {layer} pass {ps}")
