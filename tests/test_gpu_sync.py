"""The per-head synchronisation records that let the write, the query preparation and the delta
rotation each run as one launch (every work-group of a head meets at a record in the workspace
for the head's absmax).  Their contract: a workspace zero-filled once serves every later call,
whatever the sequence of operations and ring shapes sharing it, graph replays included; after
every call each record's count is back at zero, and no wait ever runs into its bound.  Results
are checked here only against the same calls made with the binding's own workspace; the parity
tests check them against the oracle."""

import pytest

from workloads import normal_bf16, tensor_seed
from kvhelpers import to_dev_bf16

pytestmark = pytest.mark.gpu

MAX_HEADS, RECORD_BYTES = 512, 6 * 128
# after the records and the error word: the split rows' arrival and departure counts of the
# attention (two 128-byte lines for each of up to 256 work-groups)
MERGE_OFFSET, MERGE_BYTES = 2 * MAX_HEADS * RECORD_BYTES + 256, 256 * 2 * 128


def _counts_zero(ws):
    """Every record's count word (the first int32 of each record) is zero, and so is every
    split-row count."""
    rec = ws[:2 * MAX_HEADS * RECORD_BYTES].view(2 * MAX_HEADS, RECORD_BYTES)[:, :4]
    merge = ws[MERGE_OFFSET:MERGE_OFFSET + MERGE_BYTES]
    return int(rec.count_nonzero().item()) == 0 and int(merge.count_nonzero().item()) == 0


def _ring_state(r):
    return [t.clone() for t in (r.k, r.v, r.k_scale, r.v_scale)]


def _same(a, b, what):
    import torch
    for x, y in zip(a, b):
        assert x.shape == y.shape and x.dtype == y.dtype, what
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), what


def test_shared_workspace_stays_zero_across_operations_and_shapes():
    import torch
    import fp8_ring_kv_write_amd as kv
    shapes = [(24, 5788, 128, 757), (3, 203, 64, 17), (5, 700, 128, 300)]
    need = max(kv.workspace_bytes(op, h, s, d, n) for (h, s, d, n) in shapes
               for op in (kv.OP_WRITE, kv.OP_DELTA_ROTATE, kv.OP_ATTENTION, kv.OP_WRITE_ATTEND))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for (h, s, d, n) in shapes:
        print(f"[sync] shared workspace {h}x{s}x{d} n={n}", flush=True)
        tab = torch.from_numpy(kv.rope_table(16384, d)).cuda()
        mine, ref = kv.Ring(h, s, d), kv.Ring(h, s, d)
        head, filled = 0, 0
        for c in range(4):
            k = to_dev_bf16(normal_bf16(tensor_seed("sync", h, d, c, 1), (n, h, d)))
            v = to_dev_bf16(normal_bf16(tensor_seed("sync", h, d, c, 2), (n, h, d)))
            q = to_dev_bf16(normal_bf16(tensor_seed("sync", h, d, c, 0), (n, h, d)))
            pos0 = 100 + c * n
            out_m, out_r = torch.empty_like(q), torch.empty_like(q)
            lse_m = torch.empty((h, n), dtype=torch.float32, device="cuda")
            lse_r = torch.empty_like(lse_m)
            if c % 2 == 0:   # write, then attention
                kv.kv_ring_write(mine, k, v, head, pos0, tab, workspace=ws)
                kv.kv_ring_write(ref, k, v, head, pos0, tab)
                nh, nf = (head + n) % s, min(filled + n, s)
                kv.ring_attention(mine, nh, nf, q, pos0, tab, 0.09, out=out_m, lse=lse_m, workspace=ws)
                kv.ring_attention(ref, nh, nf, q, pos0, tab, 0.09, out=out_r, lse=lse_r)
            else:            # the fused call, then a rotation
                nh, nf = (head + n) % s, min(filled + n, s)
                kv.kv_ring_write_attend(mine, k, v, head, pos0, nh, nf, q, pos0, tab, 0.09,
                                        out=out_m, lse=lse_m, workspace=ws)
                kv.kv_ring_write_attend(ref, k, v, head, pos0, nh, nf, q, pos0, tab, 0.09,
                                        out=out_r, lse=lse_r)
                kv.kv_ring_delta_rotate(mine, nh, nf, -37 * (c + 1), workspace=ws)
                kv.kv_ring_delta_rotate(ref, nh, nf, -37 * (c + 1))
            head, filled = nh, nf
            torch.cuda.synchronize()
            _same(_ring_state(mine), _ring_state(ref), f"ring after call {c}")
            _same([out_m, lse_m], [out_r, lse_r], f"attention of call {c}")
            assert _counts_zero(ws), f"a record's count left non-zero after call {c}"
    assert kv.sync_status(ws) == 0
    assert kv.sync_status() == 0


def test_rotation_and_write_replay_from_a_captured_graph():
    """A write followed by two rotations, captured once and replayed three times with eager work
    in between: every replay leaves the ring the eager calls leave, and the records' counts at
    zero."""
    import torch
    import fp8_ring_kv_write_amd as kv
    h, s, d, n = 6, 900, 128, 300
    tab = torch.from_numpy(kv.rope_table(16384, d)).cuda()
    ring = kv.Ring(h, s, d)
    for c in range(3):
        kv.kv_ring_write(ring, to_dev_bf16(normal_bf16(tensor_seed("sync_graph", c, 1), (n, h, d))),
                         to_dev_bf16(normal_bf16(tensor_seed("sync_graph", c, 2), (n, h, d))),
                         (c * n) % s, c * n, tab)
    k = to_dev_bf16(normal_bf16(tensor_seed("sync_graph", 9, 1), (n, h, d)))
    v = to_dev_bf16(normal_bf16(tensor_seed("sync_graph", 9, 2), (n, h, d)))
    ws = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, h, s, d, n), dtype=torch.uint8, device="cuda")
    snap = _ring_state(ring)

    def calls():
        kv.kv_ring_write(ring, k, v, 0, 3 * n, tab, workspace=ws)
        kv.kv_ring_delta_rotate(ring, n, s, -4000, workspace=ws)
        kv.kv_ring_delta_rotate(ring, n, s, 1234, workspace=ws)

    def restore():
        for t, x in zip((ring.k, ring.v, ring.k_scale, ring.v_scale), snap):
            t.copy_(x)

    calls()
    torch.cuda.synchronize()
    eager = _ring_state(ring)
    restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[sync] graph replay {rep}", flush=True)
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_ring_state(ring), eager, f"replay {rep}")
        assert _counts_zero(ws)
        _ = (k.float() * 2).sum().item()   # eager work between replays
    assert kv.sync_status(ws) == 0


def test_split_row_attention_replays_from_a_captured_graph():
    """Attention whose rows are split between work-groups (merged by the last one to finish),
    captured once and replayed three times with eager work in between: every replay gives the
    eager call's output bit for bit and leaves every count at zero."""
    import torch
    import fp8_ring_kv_write_amd as kv
    h, s, d, n = 6, 900, 128, 300     # 12 rows of 8 tiles: split over about 60 work-groups
    tab = torch.from_numpy(kv.rope_table(16384, d)).cuda()
    ring = kv.Ring(h, s, d)
    for c in range(3):
        kv.kv_ring_write(ring, to_dev_bf16(normal_bf16(tensor_seed("sync_attn", c, 1), (n, h, d))),
                         to_dev_bf16(normal_bf16(tensor_seed("sync_attn", c, 2), (n, h, d))),
                         (c * n) % s, c * n, tab)
    q = to_dev_bf16(normal_bf16(tensor_seed("sync_attn", 9, 0), (n, h, d)))
    ws = torch.zeros(kv.workspace_bytes(kv.OP_ATTENTION, h, s, d, n), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((h, n), dtype=torch.float32, device="cuda")

    def call():
        kv.ring_attention(ring, 0, s, q, 2 * n, tab, 0.088, out=out, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = [out.clone(), lse.clone()]
    assert _counts_zero(ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[sync] attention graph replay {rep}", flush=True)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same([out, lse], eager, f"attention replay {rep}")
        assert _counts_zero(ws)
        _ = (q.float() * 2).sum().item()   # eager work between replays
    assert kv.sync_status(ws) == 0


def test_a_wait_past_its_bound_is_reported_and_cleared_by_zero_fill():
    """The failure path of the per-head meeting, forced from the host: a zero-filled workspace
    whose head-0 record holds a stale count of 7 (which no call leaves behind), so the single
    work-group of a small write never finds itself the last to count in.  It polls until its
    bound (2^20 polls, about a second), sets the workspace's error word and finishes;
    kv_ring_sync_status reports it (-9).  Zero-filled again, the workspace serves the same write
    cleanly, and the ring matches one written with a fresh workspace."""
    import torch
    import fp8_ring_kv_write_amd as kv
    h, s, d, n = 1, 64, 64, 16
    tab = torch.from_numpy(kv.rope_table(16384, d)).cuda()
    k = to_dev_bf16(normal_bf16(tensor_seed("sync_bound", 0, 1), (n, h, d)))
    v = to_dev_bf16(normal_bf16(tensor_seed("sync_bound", 0, 2), (n, h, d)))
    ws = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, h, s, d, n), dtype=torch.uint8, device="cuda")
    ws[0] = 7   # the count word (first int32) of slot 0's record for head 0
    ring = kv.Ring(h, s, d)
    print("[sync] stale count: one wait runs to its bound", flush=True)
    kv.kv_ring_write(ring, k, v, 0, 0, tab, workspace=ws)
    assert kv.sync_status(ws) == -9
    ws.zero_()
    kv.kv_ring_write(ring, k, v, 0, 0, tab, workspace=ws)
    ref = kv.Ring(h, s, d)
    kv.kv_ring_write(ref, k, v, 0, 0, tab)
    torch.cuda.synchronize()
    _same(_ring_state(ring), _ring_state(ref), "the write after the zero-fill")
    assert kv.sync_status(ws) == 0
    assert _counts_zero(ws)
