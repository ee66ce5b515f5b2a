"""Parity of the three-axis rotary variant (frame, row, column positions) with the CPU oracle,
through the C ABI.

The library's per-token cos/sin rows (kv_ring_rope_table_3d) drive the unchanged write, fused
write + attention and attention calls with position offset 0; kv_ring_delta_rotate_3d moves
the cache by an offset triple.  Bars as for the 1-D path: codes and scales bit-exact,
attention within 2e-2 infinity-norm relative error per head and 1e-3 on the LSE."""

import math

import numpy as np
import pytest

import oracle
from workloads import normal_bf16, raster_positions, tensor_seed

from kvhelpers import ring_to_host, to_dev_bf16, bf16_dev_to_f64, attention_errors

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def torch():
    import torch
    return torch


@pytest.fixture(scope="module")
def kv():
    import fp8_ring_kv_write_amd as kv
    return kv


def rows(kv, torch, pos, d, bands=None):
    """Device rows from the library, host rows from the oracle; the two must be equal."""
    host = kv.rope_table_3d(pos, d, bands)
    ref = oracle.rope_rows_3d(pos, d, bands)
    assert host.tobytes() == ref.tobytes()
    return torch.from_numpy(host).cuda(), ref


class Ring3:
    """The same ring in the library (GPU) and in the oracle (CPU), written with 3-axis rows."""

    def __init__(self, kv, torch, heads, slots, d, bands=None):
        self.kv, self.torch, self.bands = kv, torch, bands
        self.g = kv.Ring(heads, slots, d)
        self.o = oracle.OracleRing(heads, slots, d)
        self.head, self.filled = 0, 0

    def write(self, k, v, start, pos):
        dev, ref = rows(self.kv, self.torch, pos, self.o.head_dim, self.bands)
        self.kv.kv_ring_write(self.g, to_dev_bf16(k), to_dev_bf16(v), start, 0, dev)
        oracle.ring_write(self.o, k, v, start, 0, ref)
        self.head, self.filled = oracle.advance(start, k.shape[0], self.filled, self.o.slots)

    def write_attend(self, k, v, start, pos, q, scale, heads):
        """Fused call: the new tokens and the queries share positions and rows."""
        dev, ref = rows(self.kv, self.torch, pos, self.o.head_dim, self.bands)
        head, filled = oracle.advance(start, k.shape[0], self.filled, self.o.slots)
        out, lse = self.kv.kv_ring_write_attend(self.g, to_dev_bf16(k), to_dev_bf16(v), start, 0,
                                                head, filled, to_dev_bf16(q), 0, dev, scale)
        self.torch.cuda.synchronize()
        oracle.ring_write(self.o, k, v, start, 0, ref)
        self.head, self.filled = head, filled
        ro, rl = oracle.ring_attention(self.o, head, filled, q, 0, ref, scale, heads=heads)
        return bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl

    def rotate(self, delta):
        self.kv.kv_ring_delta_rotate_3d(self.g, self.head, self.filled, delta, self.bands)
        oracle.ring_delta_rotate_3d(self.o, self.head, self.filled, delta, self.bands)

    def attend(self, q, qpos, scale, heads=None):
        dev, ref = rows(self.kv, self.torch, qpos, self.o.head_dim, self.bands)
        out, lse = self.kv.ring_attention(self.g, self.head, self.filled, to_dev_bf16(q), 0, dev, scale)
        self.torch.cuda.synchronize()
        ro, rl = oracle.ring_attention(self.o, self.head, self.filled, q, 0, ref, scale, heads=heads)
        return bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl

    def assert_same(self, what=""):
        self.torch.cuda.synchronize()
        k, v, ks, vs = ring_to_host(self.g)
        assert np.array_equal(k, self.o.k), f"K codes differ {what}: {np.argwhere(k != self.o.k)[:5]}"
        assert np.array_equal(v, self.o.v), f"V codes differ {what}"
        assert np.array_equal(ks, self.o.k_scale), f"K scales differ {what}"
        assert np.array_equal(vs, self.o.v_scale), f"V scales differ {what}"


def check(out, lse, ro, rl, heads, label):
    inf_rel, l2_rel = attention_errors(out[:, heads], ro[:, heads])
    dl = np.abs(lse[heads] - rl[heads])
    print(f"[{label}] inf-rel max {inf_rel.max():.2e}, L2-rel max {l2_rel.max():.2e}, "
          f"lse abs max {dl.max():.2e}", flush=True)
    assert np.all(np.isfinite(out[:, heads]))
    assert inf_rel.max() <= ATT_TOL and dl.max() <= LSE_TOL


def test_three_axis_steady_ring_reset_and_attention_full_size(kv, torch):
    """24 heads x d128 x 5,788 slots filled by 8 chunks of 757 tokens walking 22 x 34 frames
    (the last chunk through the fused write + attention call); a frame reset (-5, 0, 0); then
    757 queries at the last chunk's moved positions."""
    H, S, D, N = 24, 5788, 128, 757
    heads = [0, 7, 13, 23]
    p = Ring3(kv, torch, H, S, D)
    scale = 1 / math.sqrt(D)
    for c in range(8):
        k = normal_bf16(tensor_seed("r3full", c, 1), (N, H, D))
        v = normal_bf16(tensor_seed("r3full", c, 2), (N, H, D))
        pos = raster_positions(N, c * N)
        if c < 7:
            p.write(k, v, (c * N) % S, pos)
        else:
            q = normal_bf16(tensor_seed("r3full", c, 0), (N, H, D))
            check(*p.write_attend(k, v, (c * N) % S, pos, q, scale, heads), heads, "3-axis fused call")
    assert (p.head, p.filled) == (268, S)
    p.assert_same("steady ring")
    p.rotate((-5, 0, 0))
    p.assert_same("after frame reset")
    q = normal_bf16(tensor_seed("r3full", 99, 0), (N, H, D))
    qpos = raster_positions(N, 7 * N) + np.array([-5, 0, 0], np.int32)
    check(*p.attend(q, qpos, scale, heads), heads, "3-axis after reset")


@pytest.mark.parametrize("d,bands,delta", [
    (128, None, (3, -2, 5)),
    (128, (20, 30, 14), (-7, 0, 1)),
    (64, None, (0, 0, 0)),
    (64, (4, 8, 20), (2, 11, -3)),
])
def test_three_axis_delta_small(kv, torch, d, bands, delta):
    """3 heads, a 203-slot ring wrapped by 5 chunks of 48 tokens walking 5 x 8 frames from
    frame 10; a move along every axis, custom band cuts, a zero triple; attention after."""
    H, S, N = 3, 203, 48
    p = Ring3(kv, torch, H, S, d, bands)
    for c in range(5):
        k = normal_bf16(tensor_seed("r3s", d, c, 1), (N, H, d))
        v = normal_bf16(tensor_seed("r3s", d, c, 2), (N, H, d))
        p.write(k, v, (c * N) % S, raster_positions(N, c * N, 5, 8, 10))
    p.assert_same("filled")
    p.rotate(delta)
    p.assert_same(f"after delta {delta}")
    q = normal_bf16(tensor_seed("r3s", d, 9, 0), (33, H, d))
    qpos = raster_positions(33, 4 * N, 5, 8, 10) + np.asarray(delta, np.int32)
    check(*p.attend(q, qpos, 1 / math.sqrt(d)), list(range(H)), f"3-axis d{d} {delta}")
