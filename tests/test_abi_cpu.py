"""Host-only checks of the C ABI (no kernel is launched): the library loads, exports every
function include/kvring.h declares, its host helpers agree with the oracle, and argument
errors are reported before anything could reach the device."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvring.h")


@pytest.fixture(scope="module")
def kv():
    import fp8_ring_kv_write_amd as kv
    return kv


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("kv_ring_write", "kv_ring_delta_rotate", "ring_attention"):
        assert n in names


def test_binding_constants_match_the_header(kv):
    """The binding's operation codes and token limit are the header's."""
    text = open(HEADER).read()
    assert re.search(r"#define KV_RING_MAX_TOKENS (\d+)", text).group(1) == str(kv.MAX_TOKENS)
    for name, value in (("WRITE", kv.OP_WRITE), ("DELTA_ROTATE", kv.OP_DELTA_ROTATE),
                        ("ATTENTION", kv.OP_ATTENTION), ("WRITE_ATTEND", kv.OP_WRITE_ATTEND)):
        assert re.search(rf"KV_RING_OP_{name} = (\d+)", text).group(1) == str(value)


def test_library_exports_every_declared_function(kv):
    lib = ctypes.CDLL(kv.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_rope_table_matches_oracle_bit_for_bit(kv):
    from oracle import rope_table
    for d in (64, 128):
        ours = kv.rope_table(300, d)
        ref = rope_table(300, d)
        assert ours.tobytes() == ref.tobytes()
    # other bases (long-context rotary bases among them), and positions far out in the table
    for base in (500.0, 500000.0, 1e6):
        assert kv.rope_table(40, 128, base).tobytes() == rope_table(40, 128, base).tobytes()
    far = kv.rope_table(16384, 64)[16300:]
    assert far.tobytes() == rope_table(16384, 64)[16300:].tobytes()


def test_rope_table_3d_matches_oracle_bit_for_bit(kv):
    from oracle import rope_rows_3d
    from workloads import raster_positions
    rng = np.random.default_rng(5)
    for d, bands in ((128, None), (64, None), (128, (40, 12, 12)), (64, (32, 0, 0))):
        # a raster walk (runs of equal coordinates) and scattered, partly negative positions
        for pos in (raster_positions(300, 700, 22, 34, 3),
                    rng.integers(-5000, 5000, size=(64, 3)).astype(np.int32)):
            ours = kv.rope_table_3d(pos, d, bands)
            assert ours.tobytes() == rope_rows_3d(pos, d, bands).tobytes()


def test_code_offsets_follow_the_documented_layout(kv):
    """The library's layout functions against the numpy reading of the kvring.h formulas, and
    each tile's offsets are a permutation of the tile's bytes."""
    from kvhelpers import code_byte_maps
    for d in (64, 128):
        kmap, vmap = code_byte_maps(d)
        for slot in (0, 1, 31, 32, 77, 127, 128, 300, 5787):
            base = (slot // 128) * 128 * d
            for c in range(0, d, 5):
                assert kv.k_offset(slot, c, d) == base + kmap[slot % 128, c]
                assert kv.v_offset(slot, c, d) == base + vmap[slot % 128, c]
        ks = sorted(kv.k_offset(u, c, d) for u in range(128) for c in range(d))
        vs = sorted(kv.v_offset(u, c, d) for u in range(128) for c in range(d))
        assert ks == list(range(128 * d)) and vs == list(range(128 * d))
    assert kv.k_offset(-1, 0, 128) == -1 and kv.k_offset(0, 128, 128) == -1
    assert kv.v_offset(0, 0, 96) == -1 and kv.v_offset(0, -1, 64) == -1


def test_sizes(kv):
    assert kv.codes_bytes(24, 5788, 128) == 24 * 46 * 128 * 128
    assert kv.codes_bytes(1, 64, 64) == 128 * 64
    assert kv.codes_bytes(0, 64, 64) == 0 and kv.codes_bytes(1, 64, 96) == 0
    for op in (kv.OP_WRITE, kv.OP_DELTA_ROTATE, kv.OP_ATTENTION, kv.OP_WRITE_ATTEND):
        assert kv.workspace_bytes(op, 24, 5788, 128, 757) > 0
        assert kv.workspace_bytes(op, 24, 5788, 128, 757) % 4 == 0
    assert kv.workspace_bytes(99, 24, 5788, 128, 757) == 0
    # every workspace starts with the synchronisation records: 2 slots x 512 heads x 768 bytes
    # plus the error word's 256 bytes
    for op in (kv.OP_WRITE, kv.OP_DELTA_ROTATE, kv.OP_ATTENTION, kv.OP_WRITE_ATTEND):
        assert kv.workspace_bytes(op, 3, 64, 64, 16) >= 786688
        assert kv.workspace_bytes(op, 513, 64, 64, 16) == 0
    assert kv.workspace_bytes(kv.OP_WRITE, 24, 5788, 128, 757) == 786688
    assert kv.workspace_bytes(kv.OP_DELTA_ROTATE, 24, 5788, 128, 0) == 786688
    assert kv.workspace_bytes(kv.OP_WRITE_ATTEND, 24, 5788, 128, 757) == \
        kv.workspace_bytes(kv.OP_ATTENTION, 24, 5788, 128, 757)


def test_status_strings(kv):
    assert kv.status_string(0) == "ok"
    for s in range(-9, 0):
        assert kv.status_string(s) != "unknown status"


def test_argument_errors_are_reported_before_any_launch(kv):
    """Fake (never dereferenced) aligned addresses: every call below must be rejected by the
    argument checks, so no kernel is enqueued."""
    from fp8_ring_kv_write_amd._lib import _Desc
    L = kv.lib
    F = 1 << 20   # an aligned fake address
    good = _Desc(F, F, F, F, 2, 64, 64)
    d = ctypes.byref
    ws = kv.workspace_bytes(kv.OP_WRITE, 2, 64, 64, 16)
    # write
    assert L.kv_ring_write(None, F, F, 16, 0, 0, F, 128, F, ws, None) == -1
    assert L.kv_ring_write(d(_Desc(0, F, F, F, 2, 64, 64)), F, F, 16, 0, 0, F, 128, F, ws, None) == -1
    assert L.kv_ring_write(d(_Desc(F, F, F, F, 2, 64, 96)), F, F, 16, 0, 0, F, 128, F, ws, None) == -3
    assert L.kv_ring_write(d(_Desc(F + 1, F, F, F, 2, 64, 64)), F, F, 16, 0, 0, F, 128, F, ws, None) == -2
    assert L.kv_ring_write(d(good), F + 2, F, 16, 0, 0, F, 128, F, ws, None) == -2
    assert L.kv_ring_write(d(good), F, F, 0, 0, 0, F, 128, F, ws, None) == -4
    assert L.kv_ring_write(d(good), F, F, 65, 0, 0, F, 128, F, ws, None) == -4
    assert L.kv_ring_write(d(good), F, F, 16, 64, 0, F, 128, F, ws, None) == -4
    assert L.kv_ring_write(d(good), F, F, 16, -1, 0, F, 128, F, ws, None) == -4
    assert L.kv_ring_write(d(good), F, F, 16, 0, 120, F, 128, F, ws, None) == -5
    assert L.kv_ring_write(d(good), F, F, 16, 0, -1, F, 128, F, ws, None) == -5
    assert L.kv_ring_write(d(good), F, F, 16, 0, 0, F, 128, None, ws, None) == -6
    assert L.kv_ring_write(d(good), F, F, 16, 0, 0, F, 128, F, ws - 4, None) == -6
    # write with the static scratch: the same checks, and calls beyond the scratch rejected
    assert L.kv_ring_write_static(None, F, F, 16, 0, 0, F, 128, None) == -1
    assert L.kv_ring_write_static(d(good), F + 2, F, 16, 0, 0, F, 128, None) == -2
    assert L.kv_ring_write_static(d(good), F, F, 65, 0, 0, F, 128, None) == -4
    assert L.kv_ring_write_static(d(good), F, F, 16, 0, 120, F, 128, None) == -5
    # rings beyond 512 heads are refused by every call (the synchronisation records), so every
    # ring a call accepts fits the static scratch
    big = _Desc(F, F, F, F, 513, 1024, 64)
    assert L.kv_ring_write_static(d(big), F, F, 544, 0, 0, F, 1024, None) == -3
    assert L.kv_ring_write(d(big), F, F, 544, 0, 0, F, 1024, F, 1 << 30, None) == -3
    assert kv.workspace_bytes(kv.OP_WRITE, 512, 1024, 64, 544) > 0
    # the status word check: arguments first (nothing read)
    assert L.kv_ring_sync_status(None, None) == -1
    assert L.kv_ring_sync_status(F + 4, None) == -2
    # delta rotate
    wr = kv.workspace_bytes(kv.OP_DELTA_ROTATE, 2, 64, 64, 0)
    assert L.kv_ring_delta_rotate(d(good), 64, 10, 5, 10000.0, F, wr, None) == -4
    assert L.kv_ring_delta_rotate(d(good), 0, 65, 5, 10000.0, F, wr, None) == -4
    assert L.kv_ring_delta_rotate(d(good), 0, 10, 5, 0.0, F, wr, None) == -3
    assert L.kv_ring_delta_rotate(d(good), 0, 10, 1 << 31, 10000.0, F, wr, None) == -5
    assert L.kv_ring_delta_rotate(d(good), 0, 10, 5, 10000.0, F, wr - 4, None) == -6
    # attention
    wa = kv.workspace_bytes(kv.OP_ATTENTION, 2, 64, 64, 16)
    assert L.ring_attention(d(good), 0, 10, None, 16, 0, F, 128, 0.125, F, F, F, wa, None) == -1
    assert L.ring_attention(d(good), 0, 10, F, -1, 0, F, 128, 0.125, F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 0, 65, F, 16, 0, F, 128, 0.125, F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 64, 10, F, 16, 0, F, 128, 0.125, F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 0, 10, F, 16, 113, F, 128, 0.125, F, F, F, wa, None) == -5
    assert L.ring_attention(d(good), 0, 10, F, 16, 0, F, 128, float("nan"), F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 0, 10, F, 16, 0, F, 128, 0.0, F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 0, 10, F, 16, 0, F, 128, -0.1, F, F, F, wa, None) == -4
    assert L.ring_attention(d(good), 0, 10, F, 16, 0, F, 128, 0.125, F + 4, F, F, wa, None) == -2
    assert L.ring_attention(d(good), 0, 10, F, 16, 0, F, 128, 0.125, F, F, F, wa - 4, None) == -6
    assert L.ring_attention(d(good), 0, 10, F, 0, 0, F, 128, 0.125, F, F, F, wa, None) == 0  # no-op
    assert L.ring_attention(d(good), 0, 10, None, 0, 0, None, 128, 0.125, None, None, None, 0, None) == 0
    # encoder
    assert L.kv_ring_fp8_encode(F, F, -1, None) == -4
    assert L.kv_ring_fp8_encode(None, F, 5, None) == -1
    assert L.kv_ring_fp8_encode(F + 4, F, 5, None) == -2
    assert L.kv_ring_fp8_encode(F, F, 0, None) == 0
    assert L.kv_ring_rope_table(None, 10, 64, 10000.0) == -1
    # three-axis table and delta rotation (host arrays for positions, bands and offsets)
    pos3 = np.zeros((4, 3), np.int32)
    out3 = np.empty((4, 32, 2), np.float32)
    good_b = np.array([12, 10, 10], np.int32)
    assert L.kv_ring_rope_table_3d(None, pos3.ctypes.data, 4, 64, None, 10000.0) == -1
    assert L.kv_ring_rope_table_3d(out3.ctypes.data, None, 4, 64, None, 10000.0) == -1
    assert L.kv_ring_rope_table_3d(out3.ctypes.data, pos3.ctypes.data, 0, 64, None, 10000.0) == -3
    assert L.kv_ring_rope_table_3d(out3.ctypes.data, pos3.ctypes.data, 4, 96, None, 10000.0) == -3
    assert L.kv_ring_rope_table_3d(out3.ctypes.data, pos3.ctypes.data, 4, 64, None, 0.0) == -3
    for bad in ([12, 10, 9], [-1, 23, 10], [33, 0, -1]):
        bb = np.array(bad, np.int32)
        assert L.kv_ring_rope_table_3d(out3.ctypes.data, pos3.ctypes.data, 4, 64, bb.ctypes.data,
                                       10000.0) == -3
        assert L.kv_ring_delta_rotate_3d(d(good), 0, 10, np.zeros(3, np.int64).ctypes.data,
                                         bb.ctypes.data, 10000.0, F, wr, None) == -3
    dl = np.array([5, 0, 0], np.int64)
    big = np.array([0, 1 << 31, 0], np.int64)
    assert L.kv_ring_delta_rotate_3d(d(good), 0, 10, None, None, 10000.0, F, wr, None) == -1
    assert L.kv_ring_delta_rotate_3d(d(good), 0, 10, big.ctypes.data, None, 10000.0, F, wr, None) == -5
    assert L.kv_ring_delta_rotate_3d(d(good), 64, 10, dl.ctypes.data, None, 10000.0, F, wr, None) == -4
    assert L.kv_ring_delta_rotate_3d(d(good), 0, 10, dl.ctypes.data, good_b.ctypes.data, 0.0, F, wr,
                                     None) == -3
    assert L.kv_ring_delta_rotate_3d(d(good), 0, 10, dl.ctypes.data, None, 10000.0, F, wr - 4, None) == -6
    # write + attention in one call: the checks of both
    wf = kv.workspace_bytes(kv.OP_WRITE_ATTEND, 2, 64, 64, 16)
    assert wf >= wa   # the write shares the attention's synchronisation records
    def wa_call(*, desc=good, k=F, n=16, start=0, pos0=0, head=16, filled=16, q=F, nq=16, qpos=0,
                ntab=128, scale=0.125, out=F, lse=F, wsp=F, wsb=wf):
        return L.kv_ring_write_attend(d(desc), k, F, n, start, pos0, head, filled, q, nq, qpos, F, ntab,
                                      scale, out, lse, wsp, wsb, None)
    assert wa_call(k=None) == -1
    assert wa_call(k=F + 2) == -2
    assert wa_call(n=0) == -4
    assert wa_call(start=64) == -4
    assert wa_call(pos0=120) == -5
    assert wa_call(head=64) == -4
    assert wa_call(filled=65) == -4
    assert wa_call(nq=-1) == -4
    assert wa_call(q=None) == -1
    assert wa_call(out=F + 2) == -2
    assert wa_call(qpos=113) == -5
    assert wa_call(scale=0.0) == -4
    assert wa_call(wsb=wf - 4) == -6
    assert wa_call(desc=_Desc(F, F, F, F, 2, 64, 96)) == -3
    # more than KV_RING_MAX_TOKENS (16,384) tokens in one write or queries in one attention call:
    # their per-head meeting would need more work-groups at once than the XCDs hold
    long_ring = _Desc(F, F, F, F, 2, 1 << 20, 64)
    ntab = 1 << 16
    assert L.kv_ring_write(d(long_ring), F, F, 16385, 0, 0, F, ntab, F, 1 << 30, None) == -4
    assert L.kv_ring_write_static(d(long_ring), F, F, 16385, 0, 0, F, ntab, None) == -4
    assert L.ring_attention(d(long_ring), 0, 10, F, 16385, 0, F, ntab, 0.125, F, F, F, 1 << 30, None) == -4
    assert wa_call(desc=long_ring, n=16385, ntab=ntab, wsb=1 << 30) == -4
    assert wa_call(desc=long_ring, nq=16385, ntab=ntab, wsb=1 << 30) == -4
    assert wa_call(desc=long_ring, n=16384, nq=16384, ntab=ntab, pos0=ntab) == -5   # checks pass up to the positions
    # window copy of the read-time baseline (src, dst, fresh: 10 rows of 64 bytes each)
    S0, D0, N0 = F, F + (1 << 16), F + (2 << 16)
    assert L.kv_window_advance(S0, D0, N0, 0, 0, 64, None) == -4
    assert L.kv_window_advance(S0, D0, N0, 10, 11, 64, None) == -4
    assert L.kv_window_advance(S0, D0, N0, 10, -1, 64, None) == -4
    assert L.kv_window_advance(S0, D0, N0, 10, 3, 8, None) == -3
    assert L.kv_window_advance(S0, D0, N0, 10, 3, 72, None) == -3
    assert L.kv_window_advance(S0, None, N0, 10, 3, 64, None) == -1
    assert L.kv_window_advance(None, D0, N0, 10, 3, 64, None) == -1
    assert L.kv_window_advance(S0, D0, None, 10, 3, 64, None) == -1
    assert L.kv_window_advance(S0, D0 + 8, N0, 10, 3, 64, None) == -2
    assert L.kv_window_advance(S0, S0 + 64, N0, 10, 3, 64, None) == -4    # dst overlaps src
    assert L.kv_window_advance(S0, D0, D0 + 320, 10, 3, 64, None) == -4   # fresh inside dst


def test_product_path_has_no_oracle_import():
    """The package never imports the oracle (the oracle is test infrastructure)."""
    pkg = os.path.join(ROOT, "fp8_ring_kv_write_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_lds_copies_carry_hazard_wait_states(tmp_path):
    """The attention kernel's asynchronous global->LDS copies are inline assembly, around which
    the compiler inserts no hazard wait states: a base-address SGPR written by a vector
    instruction right before (a spilled SGPR restored with v_readlane) needs 5 wait states
    before the copy reads it.  Every copy in the generated gfx950 code must carry them."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "fp8_ring_kv_write_amd", "csrc", "ring_attention.hip")
    out = tmp_path / "ra.s"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-mllvm", "-amdgpu-mfma-vgpr-form", "-S", "--cuda-device-only", src,
                    "-o", str(out)], check=True, capture_output=True)
    lines = [l.strip() for l in out.read_text().splitlines()]
    copies = [i for i, l in enumerate(lines) if l.startswith("global_load_lds")]
    assert copies, "no LDS copies found"
    for i in copies:
        prev = [l for l in lines[max(0, i - 3):i] if l and not l.startswith(";")]
        assert prev and prev[-1] == "s_nop 4", lines[i - 3:i + 1]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with status 2 and a message, before any
    device is touched."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_binding_rejects_tensors_the_kernels_would_overrun(kv):
    """The binding checks every tensor's dtype, shape, layout and device before it hands the
    pointer to the library (which trusts it): a wrong head count, head_dim or rotary table
    would make the kernels read or write past the tensor.  Host tensors stand in for device ones
    here, and a ring on the device, so every call below must raise before the library is
    called."""
    import types
    import torch
    ring = types.SimpleNamespace(heads=2, slots=64, head_dim=64, device=torch.device("cuda"), desc=None)
    k = torch.zeros((16, 2, 64), dtype=torch.bfloat16)
    q = torch.zeros((8, 2, 64), dtype=torch.bfloat16)
    rope = torch.zeros((128, 32, 2), dtype=torch.float32)
    bad_calls = [
        lambda: kv.kv_ring_write(ring, k.float(), k, 0, 0, rope),                 # dtype
        lambda: kv.kv_ring_write(ring, k[:, :1].contiguous(), k, 0, 0, rope),     # head count
        lambda: kv.kv_ring_write(ring, k, torch.zeros((16, 2, 32), dtype=torch.bfloat16), 0, 0, rope),
        lambda: kv.kv_ring_write(ring, k.transpose(1, 2), k, 0, 0, rope),         # layout
        lambda: kv.kv_ring_write(ring, k, k, 0, 0, rope),                         # device
        lambda: kv.kv_ring_write(ring, k, k, 0, 0, torch.zeros((128, 64, 2))),    # table width
        lambda: kv.kv_ring_write_static(ring, k, k[:8], 0, 0, rope),              # token counts
        lambda: kv.ring_attention(ring, 0, 16, q.half(), 0, rope, 0.125),
        lambda: kv.ring_attention(ring, 0, 16, q, 0, rope, 0.125, out=torch.empty((4, 2, 64), dtype=torch.bfloat16)),
        lambda: kv.ring_attention(ring, 0, 16, q, 0, rope, 0.125, lse=torch.empty((2, 4))),
        lambda: kv.kv_ring_write_attend(ring, k, k, 0, 0, 16, 16, q[:, :1], 0, rope, 0.125),
        lambda: kv.kv_ring_delta_rotate(ring, 0, 16, 5, workspace=torch.zeros(64, dtype=torch.uint8)),
        lambda: kv.fp8_encode(torch.zeros(16)),                                   # host tensor
    ]
    for i, call in enumerate(bad_calls):
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"call {i} was not rejected")
