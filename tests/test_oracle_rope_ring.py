"""Pins for the oracle's rotary embedding and ring bookkeeping (CPU only)."""

import collections
import json
import math
import os

import numpy as np
import pytest

from oracle import rope_rotate, rope_table, rope_theta, valid_slots, write_slots, advance
from oracle.rope import delta_cos_sin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ring_tiny_schedule.json")


# ---------------------------------------------------------------- rotary embedding

def test_position_zero_is_exact_identity():
    t = rope_table(4, 128)
    x = np.random.default_rng(0).standard_normal((5, 128)).astype(np.float32)
    assert np.array_equal(rope_rotate(x, t[0, :, 0], t[0, :, 1]), x)


def test_rotation_is_complex_multiplication():
    # The pair (x_{2i}, x_{2i+1}) as x + iy is multiplied by exp(i p theta_i); theta_0 = 1 rad.
    d, base = 64, 10000.0
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, d)).astype(np.float32)
    pos = np.array([0, 1, 2, 17, 95, 1000, 16383])
    t = rope_table(16384, d, base)
    got = rope_rotate(x, t[pos, :, 0], t[pos, :, 1]).astype(np.float64)
    z = x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2].astype(np.float64)
    freqs = base ** (-np.arange(0, d, 2) / d)
    ref = z * np.exp(1j * pos[:, None] * freqs[None, :])
    err = np.abs(got[:, 0::2] - ref.real) + np.abs(got[:, 1::2] - ref.imag)
    assert err.max() < 4e-6 * np.abs(x).max()


def test_theta_geometric_progression():
    d = 128
    th = np.array([rope_theta(i, d) for i in range(d // 2)])
    assert th[0] == 1.0
    assert np.allclose(th[1:] / th[:-1], 10000.0 ** (-2.0 / d), rtol=1e-13, atol=0)


def test_composition_r_p_r_d_equals_r_p_plus_d():
    d = 128
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, d))
    for p, dd in [(5, 7), (1000, -400), (6212, -4000), (123, 0)]:
        # exact composition in float64 of the angle function
        a_p = np.array([p * rope_theta(i, d) for i in range(d // 2)])
        a_d = np.array([dd * rope_theta(i, d) for i in range(d // 2)])
        a_s = np.array([(p + dd) * rope_theta(i, d) for i in range(d // 2)])
        z = x[:, 0::2] + 1j * x[:, 1::2]
        two = z * np.exp(1j * a_p) * np.exp(1j * a_d)
        one = z * np.exp(1j * a_s)
        assert np.abs(two - one).max() < 1e-12 * max(1, abs(p) + abs(dd))
        # the float32 path: table at p, then delta table, vs table at p + d
        cp, sp = delta_cos_sin(p, d)
        cd, sd = delta_cos_sin(dd, d)
        cs, ss = delta_cos_sin(p + dd, d)
        x32 = x.astype(np.float32)
        r2 = rope_rotate(rope_rotate(x32, cp, sp), cd, sd)
        r1 = rope_rotate(x32, cs, ss)
        assert np.abs(r2 - r1).max() < 2e-6 * np.abs(x32).max() * math.sqrt(2)


def test_rotation_preserves_pair_norms_and_relative_dot_products():
    d = 128
    rng = np.random.default_rng(3)
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    t = rope_table(16384, d)
    qr = rope_rotate(q, t[700, :, 0], t[700, :, 1]).astype(np.float64)
    assert np.allclose(qr[0::2] ** 2 + qr[1::2] ** 2, q.astype(np.float64)[0::2] ** 2 + q.astype(np.float64)[1::2] ** 2,
                       rtol=1e-6)
    dots = []
    for shift in [0, 11, 4000]:
        a = rope_rotate(q, t[700 + shift, :, 0], t[700 + shift, :, 1]).astype(np.float64)
        b = rope_rotate(k, t[650 + shift, :, 0], t[650 + shift, :, 1]).astype(np.float64)
        dots.append(a @ b)
    assert np.allclose(dots, dots[0], rtol=0, atol=1e-4)


def test_table_matches_angle_function_rounded_once():
    t = rope_table(64, 64)
    for p in [0, 1, 33, 63]:
        for i in [0, 5, 31]:
            a = p * 10000.0 ** (-(2.0 * i) / 64)
            assert t[p, i, 0] == np.float32(math.cos(a))
            assert t[p, i, 1] == np.float32(math.sin(a))


# ---------------------------------------------------------------- ring bookkeeping

def test_ring_matches_linear_window_bruteforce():
    """The ring's valid slots, oldest first, hold exactly the last `filled` tokens of a plain
    sliding window (a deque with maxlen S), for every S <= 20 and every write size, over
    histories long enough to wrap several times."""
    for S in range(1, 21):
        for n in range(1, S + 1):
            window = collections.deque(maxlen=S)
            slot_token = [-1] * S
            head, filled, tok = 0, 0, 0
            for _ in range(2 * S // n + 3):
                for i, s in enumerate(write_slots(head, n, S)):
                    slot_token[s] = tok + i
                window.extend(range(tok, tok + n))
                tok += n
                head, filled = advance(head, n, filled, S)
                got = [slot_token[s] for s in valid_slots(head, filled, S)]
                assert got == list(window), (S, n)


def test_every_slot_count_start_and_write_size():
    """Exhaustive over S <= 64, every start slot and every write size n <= S, from four prior
    fill levels (empty, one token, half, full): a token-by-token simulation (each token goes to
    the slot after the previous one, wrapping at S) gives the write's slots, and the valid slots
    after the write are those holding the newest min(filled + n, S) tokens, oldest first."""
    for S in range(1, 65):
        for start in range(S):
            for f0 in sorted({0, min(1, S), S // 2, S}):
                # the f0 tokens before the write sit in the f0 slots just before `start`
                owner = [-1] * S
                for j in range(f0):
                    owner[(start - f0 + j) % S] = j
                for n in range(1, S + 1):
                    sim, s = [], start
                    for _ in range(n):
                        sim.append(s)
                        s = s + 1 if s + 1 < S else 0
                    got = write_slots(start, n, S)
                    assert list(got) == sim, (S, start, n)
                    own = owner[:]
                    for i, slot in enumerate(sim):
                        own[slot] = f0 + i
                    keep = min(f0 + n, S)
                    newest = sorted((t, slot) for slot, t in enumerate(own) if t >= f0 + n - keep)
                    head, filled = advance(start, n, f0, S)
                    assert (head, filled) == (s, keep), (S, start, n, f0)
                    assert list(valid_slots(head, filled, S)) == [slot for _, slot in newest], (S, start, n, f0)


def test_tiny_schedule_golden():
    g = json.load(open(GOLDEN))
    S, n = g["slots"], g["n"]
    filled = 0
    for w in g["writes"]:
        slots = write_slots(w["start"], n, S)
        assert slots[0] == w["start"] and slots[-1] == (w["start"] + n - 1) % S
        head, filled = advance(w["start"], n, filled, S)
        assert (head, filled) == (w["head_after"], w["filled_after"])
        vs = valid_slots(head, filled, S)
        assert (vs[0], vs[-1]) == (w["valid_first"], w["valid_last"])
    ex = g["wrap_example"]
    s = write_slots(ex["start"], ex["n"], ex["slots"])
    runs = [s[s >= ex["start"]], s[s < ex["start"]]]
    assert [runs[0][0], runs[0][-1]] == ex["first_run"]
    assert [runs[1][0], runs[1][-1]] == ex["second_run"]


def test_ring_argument_errors():
    with pytest.raises(ValueError):
        write_slots(64, 1, 64)
    with pytest.raises(ValueError):
        write_slots(0, 65, 64)
    with pytest.raises(ValueError):
        valid_slots(0, 65, 64)
