"""Pins for the oracle's three-axis rotary positions (frame, row, column) and the delta rotation
that moves one axis, CPU only.

What pins what:
* the cos/sin rows: each band, read on its own, is bit for bit the 1-D table (itself pinned by
  composition, orthogonality and the identity at position 0) of dimension twice the band's
  pairs at that band's coordinate; with one band holding every pair the rows are the 1-D
  table; zero coordinates leave their bands unrotated exactly; negative coordinates mirror
  positive ones (cos even, sin odd);
* relative positions: a score between a rotated query and a rotated key is unchanged when both
  move by the same triple, and changes when the query moves along any single axis;
* the 3-axis delta: with one band holding every pair it is the 1-D delta bit for bit; a frame
  reset equals writing the keys at the shifted frames up to the first write's FP8 error and
  leaves the row and column channels exactly as dequantised; a zero triple keeps the codes of a
  single-write ring; attention is unchanged (within the quantisation error) when keys and
  queries move together, and far off when the wrong axis is moved.
"""

import numpy as np
import pytest

from oracle import (OracleRing, advance, band_of_pairs, default_bands, delta_cos_sin_3d,
                    ring_attention, ring_delta_rotate_3d, ring_write, rope_rotate, rope_rows_3d,
                    rope_table, valid_slots)
from oracle.fp8 import e4m3_decode
from oracle.kvcache import dequant_ring, softmax_attention, widen_bf16
from oracle.rope import delta_cos_sin
from workloads import normal_bf16, raster_positions, tensor_seed


def test_default_band_cut():
    assert default_bands(128) == (22, 21, 21)
    assert default_bands(64) == (12, 10, 10)
    band, local, size = band_of_pairs(128)
    assert list(np.bincount(band)) == [22, 21, 21]
    assert (local[0], local[21], local[22], local[43], local[63]) == (0, 21, 0, 0, 20)
    assert set(size[band == 1]) == {21}
    for bad in [(22, 21, 20), (-1, 33, 32), (64, 0), (30, 30, 5)]:
        with pytest.raises(ValueError):
            band_of_pairs(128, bad)


@pytest.mark.parametrize("d,bands", [(128, None), (64, None), (128, (32, 16, 16)),
                                     (64, (0, 16, 16)), (128, (64, 0, 0)), (64, (1, 30, 1))])
def test_each_band_is_a_1d_table_of_its_own_dimension(d, bands):
    rng = np.random.default_rng(d + (0 if bands is None else sum(bands[:1])))
    pos = rng.integers(0, 100, size=(40, 3)).astype(np.int32)
    rows = rope_rows_3d(pos, d, bands)
    assert rows.shape == (40, d // 2, 2) and rows.dtype == np.float32
    cut = default_bands(d) if bands is None else bands
    off = 0
    for axis, p in enumerate(cut):
        if p:
            ref = rope_table(100, 2 * p)[pos[:, axis]]
            assert np.array_equal(rows[:, off:off + p], ref), axis
        off += p


def test_negative_coordinates_mirror_positive_ones():
    pos = np.array([[5, 7, 9], [0, 3, 0], [4000, 21, 33]], np.int32)
    a, b = rope_rows_3d(pos, 128), rope_rows_3d(-pos, 128)
    assert np.array_equal(b[..., 0], a[..., 0]) and np.array_equal(b[..., 1], -a[..., 1])


def test_zero_coordinates_leave_their_bands_unrotated():
    rows = rope_rows_3d(np.array([[0, 0, 0], [9, 0, 0], [0, 4, 0], [0, 0, 3]], np.int32), 128)
    band, _, _ = band_of_pairs(128)
    assert np.all(rows[0, :, 0] == 1) and np.all(rows[0, :, 1] == 0)
    for r, axis in ((1, 0), (2, 1), (3, 2)):
        still = band != axis
        assert np.all(rows[r, still, 0] == 1) and np.all(rows[r, still, 1] == 0)
        assert np.all(rows[r, ~still, 1] != 0)


def _rot(x, rows):
    """float64 rotation of x[..., D] by float32 rows[..., D/2, 2] (widened exactly)."""
    c, s = rows[..., 0].astype(np.float64), rows[..., 1].astype(np.float64)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def test_scores_depend_on_position_differences_only():
    rng = np.random.default_rng(3)
    d = 128
    q, k = rng.standard_normal((60, d)), rng.standard_normal((60, d))
    a, b = rng.integers(0, 40, (60, 3)), rng.integers(0, 40, (60, 3))
    norm = np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1)

    def score(qp, kp):
        return (_rot(q, rope_rows_3d(qp, d)) * _rot(k, rope_rows_3d(kp, d))).sum(-1)

    base = score(a, b)
    for shift in ([7, 3, 11], [-30, 0, 2], [0, 25, 0]):
        moved = score(a + np.array(shift), b + np.array(shift))
        assert np.all(np.abs(moved - base) <= 1e-5 * norm)   # float32 cos/sin rounding only
    for axis in range(3):
        e = np.zeros(3, np.int64)
        e[axis] = 1
        assert np.abs(score(a + e, b) - base).max() > 1e-2 * norm.max()


@pytest.mark.parametrize("d", [64, 128])
def test_delta_3d_with_one_band_is_the_1d_delta(d):
    for delta in (0, 1, -4000, 12345):
        c, s = delta_cos_sin_3d((delta, 5, -7), d, (d // 2, 0, 0))
        c1, s1 = delta_cos_sin(delta, d)
        assert np.array_equal(c, c1) and np.array_equal(s, s1)


H, D, S, N, ROWS, COLS, T0 = 2, 64, 150, 60, 5, 8, 30


def _ring3d(writes=3, name="r3"):
    """A ring filled by `writes` chunks of N tokens walking a raster of ROWS x COLS frames from
    frame T0; returns the ring, its head and fill, and the raw keys/values and positions of
    every slot."""
    ring = OracleRing(H, S, D)
    raw_k = np.zeros((H, S, D), np.float32)
    raw_v = np.zeros((H, S, D), np.float32)
    pos = np.zeros((S, 3), np.int64)
    head, filled = 0, 0
    for c in range(writes):
        p = raster_positions(N, c * N, ROWS, COLS, T0)
        k = normal_bf16(tensor_seed(name, c, 1), (N, H, D))
        v = normal_bf16(tensor_seed(name, c, 2), (N, H, D))
        start = (c * N) % S
        ring_write(ring, k, v, start, 0, rope_rows_3d(p, D))
        sl = (start + np.arange(N)) % S
        raw_k[:, sl] = widen_bf16(k).transpose(1, 0, 2)
        raw_v[:, sl] = widen_bf16(v).transpose(1, 0, 2)
        pos[sl] = p
        head, filled = advance(start, N, filled, S)
    return ring, head, filled, raw_k, raw_v, pos


def test_frame_reset_equals_writing_at_shifted_frames():
    ring, head, filled, raw_k, _, pos = _ring3d()
    assert filled == S                       # three chunks of 60 wrap a 150-slot ring
    before = ring.copy()
    delta = np.array([-25, 0, 0])
    k_rot = ring_delta_rotate_3d(ring, head, filled, delta)
    vs = valid_slots(head, filled, S)
    rows = rope_rows_3d(pos[vs] + delta, D)
    ref = rope_rotate(raw_k[:, vs], rows[None, :, :, 0], rows[None, :, :, 1])
    amax = np.abs(ref).max(axis=(1, 2))
    assert np.all(np.abs(k_rot - ref).max(axis=(1, 2)) <= amax * 2 ** -4 * 1.5)
    _, k_hat, _ = dequant_ring(ring, head, filled)
    assert np.all(np.abs(k_hat - ref).max(axis=(1, 2)) <= amax * 2 ** -3 * 1.5)
    # the row and column channels are exactly the dequantised keys; the frame channels move
    band, _, _ = band_of_pairs(D)
    ch = np.repeat(band, 2)
    deq = e4m3_decode(before.k[:, vs]).astype(np.float32) * before.k_scale[:, vs, None]
    assert np.array_equal(k_rot[..., ch != 0], deq[..., ch != 0])
    assert np.abs(k_rot[..., ch == 0] - deq[..., ch == 0]).max() > 0.1 * amax.min()
    assert np.array_equal(ring.v, before.v) and np.array_equal(ring.v_scale, before.v_scale)


def test_zero_triple_keeps_the_codes_of_a_single_write_ring():
    ring, head, filled, _, _, _ = _ring3d(writes=1)
    before = ring.copy()
    ring_delta_rotate_3d(ring, head, filled, (0, 0, 0))
    assert np.array_equal(ring.k, before.k)
    vs = valid_slots(head, filled, S)
    assert np.all(np.abs(ring.k_scale[:, vs] - before.k_scale[:, vs]) <= np.spacing(before.k_scale[:, vs]))


def _rot64_3d(x, pos, d):
    """float64 three-band rotation from the band definition (complex exponentials)."""
    band, local, size = band_of_pairs(d)
    freqs = np.power(10000.0, -local / size)
    ang = pos[:, band].astype(np.float64) * freqs[None, :]
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def test_frame_reset_preserves_attention_when_queries_move_too():
    ring, head, filled, raw_k, raw_v, pos = _ring3d()
    nq = 40
    q = normal_bf16(tensor_seed("r3q", 0), (nq, H, D))
    qpos = raster_positions(nq, 2 * N, ROWS, COLS, T0).astype(np.int64)
    vs = valid_slots(head, filled, S)
    exact = np.zeros((nq, H, D))
    for h in range(H):
        qh = _rot64_3d(widen_bf16(q)[:, h].astype(np.float64), qpos, D)
        kh = _rot64_3d(raw_k[h, vs].astype(np.float64), pos[vs], D)
        exact[:, h], _ = softmax_attention(qh, kh, raw_v[h, vs].astype(np.float64), 0.125)

    def rel(o):
        return (np.abs(o - exact).max(axis=(0, 2)) / np.abs(exact).max(axis=(0, 2))).max()

    out0, _ = ring_attention(ring, head, filled, q, 0, rope_rows_3d(qpos, D), 0.125)
    for delta, close in (((-25, 0, 0), True), ((0, -3, 0), True), ((-25, 0, 0), False)):
        d = np.array(delta)
        moved = ring.copy()
        ring_delta_rotate_3d(moved, head, filled, d)
        # queries move with the keys, or (close=False) along the wrong axis
        qd = d if close else np.array([0, -25, 0])
        out1, _ = ring_attention(moved, head, filled, q, 0, rope_rows_3d(qpos + qd, D), 0.125)
        if close:
            assert rel(out1) < 2 * rel(out0) + 0.02, delta
        else:
            assert rel(out1) > 0.3
    assert rel(out0) < 0.1
