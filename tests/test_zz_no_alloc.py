"""kv_ring_write_static -- the write for callers that cannot allocate, with the library's static
device scratch instead of a workspace -- against kv_ring_write on the same inputs: identical ring
codes and scales after each of two calls in a row, the second smaller than the first (the
scratch keeps the first call's contents, which the second must not depend on)."""

import numpy as np
import pytest

from workloads import normal_bf16, tensor_seed

from kvhelpers import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("heads,slots,d,calls", [
    (24, 5788, 128, [(2894, 5000, 100), (757, 268, 4000)]),   # wraps; then the steady-state write
    (3, 203, 64, [(203, 7, 0), (17, 190, 300)]),
])
def test_static_scratch_write_matches_workspace_write(heads, slots, d, calls):
    import torch
    import fp8_ring_kv_write_amd as kv
    tab = torch.from_numpy(kv.rope_table(16384, d)).cuda()
    ref, got = kv.Ring(heads, slots, d), kv.Ring(heads, slots, d)
    for j, (n, start, pos0) in enumerate(calls):
        print(f"[static write] {heads}x{slots}x{d} call {j}: n={n} start={start}", flush=True)
        k = to_dev_bf16(normal_bf16(tensor_seed("static_write", d, j, 1), (n, heads, d)))
        v = to_dev_bf16(normal_bf16(tensor_seed("static_write", d, j, 2), (n, heads, d)))
        kv.kv_ring_write(ref, k, v, start, pos0, tab)
        kv.kv_ring_write_static(got, k, v, start, pos0, tab)
        torch.cuda.synchronize()
        for a, b in ((ref.k, got.k), (ref.v, got.v), (ref.k_scale, got.k_scale), (ref.v_scale, got.v_scale)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"call {j} differs"
