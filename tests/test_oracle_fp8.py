"""Pins for the oracle's E4M3 codec (CPU only).

The codec is pinned to the OCP format definition's landmark values (golden fixture), to
torch's own float8_e4m3fn conversion (an independent library routine, which rounds to
nearest-even but turns overflow into NaN instead of saturating), and to an exact
rational brute force on sampled inputs including every tie."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_decode_table, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_landmarks.json")


def test_decode_landmarks_from_spec():
    spec = json.load(open(GOLDEN))
    for code_s, val in spec["codes"].items():
        code = int(code_s, 16)
        got = e4m3_decode(np.array([code], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code_s
        else:
            assert got == float(val), code_s
            assert np.signbit(got) == np.signbit(float(val)), code_s


def test_decode_table_matches_torch_all_codes():
    ours = e4m3_decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], theirs[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(theirs[fin]))


def _torch_encode(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _grid_points_and_neighbours() -> np.ndarray:
    """Every representable value, every midpoint, and the float32 neighbours of each."""
    pos = e4m3_decode_table()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    base = np.concatenate([pos, mids, [464.0]]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    pts = np.concatenate([base, up, dn])
    pts = pts[pts >= 0]
    return np.concatenate([pts, -pts]).astype(np.float32)


def test_encode_matches_torch_on_grid_and_midpoints():
    x = _grid_points_and_neighbours()
    x = x[np.abs(x) <= 464.0]  # torch's conversion turns overflow into NaN; in range it is RNE
    assert np.array_equal(e4m3_encode(x), _torch_encode(x))


def test_encode_matches_torch_on_strided_float32_sweep():
    # every 61st float32 bit pattern with magnitude in [0, 464]: ~1.1e7 values in 2 signs
    top = np.float32(464.0).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 61, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.concatenate([x, -x])
    for chunk in np.array_split(x, 8):
        assert np.array_equal(e4m3_encode(chunk), _torch_encode(chunk))


def _exact_nearest(x: float) -> int:
    """Brute force over all 127 non-negative codes with exact rational distances."""
    table = e4m3_decode_table()
    a = min(abs(Fraction(float(x))), Fraction(448))
    best = None
    for code in range(0x7F):
        d = abs(Fraction(float(table[code])) - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    sign = 0x80 if np.signbit(x) else 0
    return best[1] | sign


def test_encode_exact_bruteforce_sample():
    rng = np.random.default_rng(7)
    samples = np.concatenate([
        _grid_points_and_neighbours()[::7],
        (rng.standard_normal(300) * 50).astype(np.float32),
        (rng.uniform(0, 2 ** -6, 200)).astype(np.float32),
        np.array([1000.0, -1e30, 449.0, 2 ** -10, -2 ** -10, 3 * 2 ** -11, 0.0, -0.0], np.float32),
    ]).astype(np.float32)
    got = e4m3_encode(samples)
    for x, g in zip(samples.tolist(), got.tolist()):
        assert g == _exact_nearest(np.float32(x)), x


def test_encode_saturates_and_keeps_sign_of_zero():
    x = np.array([448.0, 460.0, 464.0, 470.0, 1e30, -1e30, -0.0, 0.0, -1e-30], np.float32)
    assert e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


def test_roundtrip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)
