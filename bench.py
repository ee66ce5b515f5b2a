#!/usr/bin/env python3
"""Benchmark of the write-time FP8 ring KV-cache hot path on one MI355X.

One step = one layer call of the path, the unit the Runway Characters pages count 240 of per
chunk (abstract of arXiv 2611.05642): kv_ring_write of 757 new tokens (RoPE + per-head FP8)
into a full 5,788-slot ring, then ring_attention of 757 queries over all 5,788 slots, with 24
heads x head_dim 128 as one GPU's share, issued as one kv_ring_write_attend call (the same
work and results as the two calls; the two-call step is timed and reported beside it).  Inputs
are seeded synthetic N(0,1) bfloat16 tensors already resident in device memory.  `value` is
steps per second, i.e. ring_attention calls per second including their write.  The GPU's clock
ramps up over a fraction of a second of sustained load, so half a second of untimed layer calls
(`clock_ramp_s`) precedes the W warm-up steps and the K timed ones, as in a serving loop.

Also reported (one JSON line on stdout; progress on stderr):
  attention   the main attention kernel alone, timed with HIP events recorded on its launch
              stream around each launch (53.84 GFLOP algorithmic per call: 4 * 757 * 5788 *
              128 * 24), as a fraction of the FP8 matrix-core peak -> the `roofline` object;
  write       kv_ring_write per call (14.10 MB algorithmic: bf16 K and V read, FP8 codes and
              per-slot scales written) as a fraction of HBM peak, from its cold-cache GPU time
              (the warm graph-replay time beside it as cache-resident throughput);
  delta_rotate kv_ring_delta_rotate of one full ring (36.67 MB algorithmic: K codes and
              scales read and written), the same way;
  launch_floor_us  GPU time of one dependent launch of a near-empty kernel (graph replays);
  reset_60_layers  the position-reset workload with outliers: 60 rings of Student-t K/V with
              x20 outlier channels, each rotated by -4,000 then attended (2.2 GB, cold);
  chunk       240 (write + attention) calls over 60 rings, 4 passes, as one chunk;
  cold_cache  write, delta rotation and step timed one call at a time after a 512 MB buffer is
              rewritten (the infinity cache no longer holds the ring, as between two calls of
              one layer in a 60-layer model);
  write_sweep kv_ring_write time and GB/s over the token count (32 .. 5,788);
  fill_up     ring_attention time over the fill level after each of the 8 writes that fill
              an empty ring (the first chunks of a session);
  three_axis  the (frame, row, column) position variant: fused step, write and frame reset
              (kv_ring_delta_rotate_3d by (-5, 0, 0)) with per-token rows, and the host time to
              build one chunk's rows (kv_ring_rope_table_3d);
  read_time_baseline  the design the ring replaces, with the same kernels: per call the linear
              bfloat16 window is copied forward by the new tokens (kv_window_advance), rotated
              and quantised whole (kv_ring_write of all 5,788 tokens), then attended; its
              cache-maintenance time per call against the ring's write;
  hbm_copy_GBps a plain 512 MiB device-to-device copy, bytes read + written per second: the
              achievable HBM line beside the 8 TB/s peak (write and delta_rotate give both
              fractions);
  cpu_baseline the CPU oracle on the same step (full call), on the host's cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring_attention calls/s at 757×5788×d128 (%FP8 MFMA peak); kv write GB/s"
H, S, D, N = 24, 5788, 128, 757
ROPE_POS = 16384
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 matrix-core peak
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E peak
ATT_FLOP = 4.0 * N * S * D * H
ATT_KERNEL = "attn_pp<128>"
# HBM bytes per launch of the main attention kernel from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) over this workload, each divided by the factor the same counter
# reads for a torch copy of --calibrate-copy bytes.  Valid only for the kernel sources whose
# hash is recorded; reported as null otherwise.
ATT_TRAFFIC = {"sources": "1ca77da08170c0dc", "bytes": 124_850_000,
               "read_bytes": 98_490_000, "write_bytes": 26_360_000}
WRITE_BYTES = 2 * N * H * D * 2 + 2 * N * H * D + 2 * N * H * 4
CLOCK_RAMP_S = 0.5            # untimed layer calls before the warm-up steps (clock ramp)
ROTATE_BYTES = 2 * (H * S * D + H * S * 4)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-chunk", action="store_true", help="skip the 240-call chunk measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-time", action="store_true", help="skip the read-time baseline")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timings")
    ap.add_argument("--no-reset", action="store_true",
                    help="skip the position-reset workload (60 outlier rings rotated, then attended)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time repeated calls as issued from Python only (no graph replays; for profilers)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the write-size and fill-up sweeps")
    ap.add_argument("--no-copy-line", action="store_true",
                    help="skip the device-copy measurement (the achievable HBM rate)")
    ap.add_argument("--no-three-axis", action="store_true",
                    help="skip the three-axis (frame, row, column) position variant")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of heads on one GPU; --gpus {args.gpus} is not "
              "supported (the path shards by heads with no exchange; see the design notes).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp8_ring_kv_write_amd as kv
    from workloads import normal_bf16, tensor_seed, steady_ring_schedule

    dev = torch.device("cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    tab = torch.from_numpy(kv.rope_table(ROPE_POS, D)).to(dev)
    ring = kv.Ring(H, S, D, dev)
    sched = steady_ring_schedule(S, N, 8)
    filled = 0
    for c, w in enumerate(sched):
        kv.kv_ring_write(ring, to_dev(normal_bf16(tensor_seed("single_call", c, 1), (N, H, D))),
                         to_dev(normal_bf16(tensor_seed("single_call", c, 2), (N, H, D))),
                         w.start_slot, w.pos0, tab)
        filled = min(filled + N, S)
    head = (sched[-1].start_slot + N) % S
    assert (head, filled) == (268, S)
    # the step rewrites the newest chunk's slots (as each denoising pass does) and attends
    start, pos0 = sched[-1].start_slot, sched[-1].pos0
    k_new = to_dev(normal_bf16(tensor_seed("single_call", 100, 1), (N, H, D)))
    v_new = to_dev(normal_bf16(tensor_seed("single_call", 100, 2), (N, H, D)))
    q = to_dev(normal_bf16(tensor_seed("single_call", 99, 0), (N, H, D)))
    scale = 1.0 / math.sqrt(D)
    ws_w = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, H, S, D, N), dtype=torch.uint8, device=dev)
    ws_a = torch.zeros(kv.workspace_bytes(kv.OP_ATTENTION, H, S, D, N), dtype=torch.uint8, device=dev)
    ws_r = torch.zeros(kv.workspace_bytes(kv.OP_DELTA_ROTATE, H, S, D, 0), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)

    if args.calibrate_copy > 0:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ws_f = torch.zeros(kv.workspace_bytes(kv.OP_WRITE_ATTEND, H, S, D, N), dtype=torch.uint8, device=dev)

    def step():
        kv.kv_ring_write_attend(ring, k_new, v_new, start, pos0, head, filled, q, pos0, tab, scale,
                                out=out, lse=lse, workspace=ws_f, stream=stream)

    def graph_us(fn, n_calls):
        """GPU time per call of fn(i) for i < n_calls, captured once in a HIP graph and replayed
        (no host work between the calls: the time the GPU needs, not the time Python needs to
        issue them).  With --no-graph: the calls issued back to back instead."""
        if args.no_graph:
            for i in range(n_calls):
                fn(i)
            e0.record(stream)
            for i in range(n_calls):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return 1000.0 * e0.elapsed_time(e1) / n_calls
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_calls):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / n_calls

    def step_separate():
        kv.kv_ring_write(ring, k_new, v_new, start, pos0, tab, workspace=ws_w, stream=stream)
        kv.ring_attention(ring, head, filled, q, pos0, tab, scale, out=out, lse=lse, workspace=ws_a,
                          stream=stream)

    # ---------------------------------------------------------------- the timed steps
    # the clock's ramp under sustained load: half a second of untimed layer calls first
    log(f"clock ramp: {CLOCK_RAMP_S} s of untimed layer calls")
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < CLOCK_RAMP_S:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = wall * 1000.0 / args.steps
    log(f"step: {ms_per_step * 1000:.1f} us wall, {gpu_ms * 1000:.1f} us GPU")
    # the same step as two calls (kv_ring_write, then ring_attention)
    for _ in range(5):
        step_separate()
    e0.record(stream)
    for _ in range(args.steps):
        step_separate()
    e1.record(stream)
    torch.cuda.synchronize()
    sep_ms = e0.elapsed_time(e1) / args.steps
    log(f"step as two calls: {sep_ms * 1000:.1f} us GPU")

    # ---------------------------------------------------------------- attention kernel alone
    reps = max(50, args.steps // 2) // 2 * 2
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for b, a in evs:        # torch creates the HIP event on its first record(); the library then
        b.record(stream)    # re-records the same events around the attention kernel
        a.record(stream)
    # the GPU's clock ramps up under sustained load: run calls for about half a second first
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.5:
        for _ in range(20):
            kv.ring_attention(ring, head, filled, q, pos0, tab, scale, out=out, lse=lse, workspace=ws_a,
                              stream=stream)
        torch.cuda.synchronize()
    for b, a in evs[:5]:
        kv.set_attention_events(b, a)
        kv.ring_attention(ring, head, filled, q, pos0, tab, scale, out=out, lse=lse, workspace=ws_a, stream=stream)
    torch.cuda.synchronize()
    for (b, a), (cb, ca) in zip(evs, calls):
        kv.set_attention_events(b, a)
        cb.record(stream)
        kv.ring_attention(ring, head, filled, q, pos0, tab, scale, out=out, lse=lse, workspace=ws_a, stream=stream)
        ca.record(stream)
    kv.set_attention_events(None, None)
    torch.cuda.synchronize()
    att_us = 1000.0 * sum(b.elapsed_time(a) for b, a in evs) / reps
    call_us = 1000.0 * sum(b.elapsed_time(a) for b, a in calls) / reps
    att_tflops = ATT_FLOP / (att_us * 1e-6) / 1e12
    log(f"attention kernel {att_us:.1f} us ({att_tflops:.0f} TFLOP/s), whole call {call_us:.1f} us")

    # ---------------------------------------------------------------- write alone
    # back to back between two events, like the steps: the throughput of repeated writes
    for _ in range(5):
        kv.kv_ring_write(ring, k_new, v_new, start, pos0, tab, workspace=ws_w, stream=stream)
    e0.record(stream)
    for _ in range(reps):
        kv.kv_ring_write(ring, k_new, v_new, start, pos0, tab, workspace=ws_w, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    write_us = 1000.0 * e0.elapsed_time(e1) / reps
    write_gpu_us = graph_us(lambda i: kv.kv_ring_write(ring, k_new, v_new, start, pos0, tab, workspace=ws_w), 50)
    write_gbps = WRITE_BYTES / (write_gpu_us * 1e-6) / 1e9
    log(f"write {write_gpu_us:.1f} us GPU ({write_gbps:.0f} GB/s), {write_us:.1f} us per call issued from Python")

    # ---------------------------------------------------------------- delta rotation of one ring
    for i in range(4):
        kv.kv_ring_delta_rotate(ring, head, filled, -4000 if i % 2 == 0 else 4000, workspace=ws_r, stream=stream)
    e0.record(stream)
    for i in range(reps):   # +-4000 alternate, so positions stay within range
        kv.kv_ring_delta_rotate(ring, head, filled, -4000 if i % 2 == 0 else 4000, workspace=ws_r, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    rot_us = 1000.0 * e0.elapsed_time(e1) / reps
    rot_gpu_us = graph_us(lambda i: kv.kv_ring_delta_rotate(ring, head, filled, -4000 if i % 2 == 0 else 4000,
                                                            workspace=ws_r), 50)
    rot_gbps = ROTATE_BYTES / (rot_gpu_us * 1e-6) / 1e9
    log(f"delta rotate {rot_gpu_us:.1f} us GPU ({rot_gbps:.0f} GB/s), {rot_us:.1f} us per call issued from Python")

    # ---------------------------------------------------------------- achievable HBM rate
    # A plain device-to-device copy of 512 MiB (twice the infinity cache, so it streams from and
    # to HBM): bytes read + written per second, the practical ceiling for the streaming kernels.
    copy_gbps = None
    if not args.no_copy_line:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2.0 * src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        log(f"device copy of 512 MiB: {copy_gbps:.0f} GB/s (read + written)")

    # ---------------------------------------------------------------- cold caches
    # Between two calls on the same layer a model runs every other layer, whose rings (60 x 36 MB)
    # push this one out of the 256 MB infinity cache.  Here a 512 MB buffer is rewritten before
    # each call to the same effect.  GPU time per call: a captured graph of (rewrite, call) x 20
    # replayed, minus a graph of the 20 rewrites alone (no host work between the calls).  The HBM
    # fractions of the write and the rotation are taken from these times; the warm replays above
    # (inputs and ring resident in the caches) are reported as cache-resident throughput only.
    cold = None
    flush = None
    if not args.no_cold:
        # rewritten by an elementwise kernel (no memset, which a captured graph should not hold)
        flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        cold_reps = 20

        def graph_ms(body, reps):
            body(0)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(reps):
                    body(i)
            gr.replay()
            torch.cuda.synchronize()
            best = None
            for _ in range(3):
                e0.record(stream)
                gr.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1)
                best = t if best is None else min(best, t)
            del gr
            return best

        flush_ms = graph_ms(lambda i: flush.add_(1.0), cold_reps)

        def timed_cold(fn):
            def body(i):
                flush.add_(1.0)
                fn(i)
            return 1000.0 * max(graph_ms(body, cold_reps) - flush_ms, 0.0) / cold_reps

        c_write = timed_cold(lambda i: kv.kv_ring_write(ring, k_new, v_new, start, pos0, tab, workspace=ws_w))
        c_rot = timed_cold(lambda i: kv.kv_ring_delta_rotate(ring, head, filled, -4000 if i % 2 == 0 else 4000,
                                                             workspace=ws_r))
        c_step = timed_cold(lambda i: kv.kv_ring_write_attend(ring, k_new, v_new, start, pos0, head, filled, q, pos0,
                                                               tab, scale, out=out, lse=lse, workspace=ws_f))
        cold = {"write_us": round(c_write, 2), "write_GBps": round(WRITE_BYTES / (c_write * 1e-6) / 1e9, 1),
                "delta_rotate_us": round(c_rot, 2),
                "delta_rotate_GBps": round(ROTATE_BYTES / (c_rot * 1e-6) / 1e9, 1),
                "step_us": round(c_step, 2), "calls": cold_reps,
                "method": "graph of (512 MB rewrite, call) x 20 minus graph of the rewrites"}
        log(f"cold caches: write {c_write:.1f} us, delta rotate {c_rot:.1f} us, step {c_step:.1f} us")

    # ---------------------------------------------------------------- the floor of one launch
    # GPU time per launch of a kernel that does almost nothing (a one-element add), replayed from a
    # captured graph like the calls above: the fixed cost every dependent launch pays on this part
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    launch_floor_us = graph_us(lambda i: tiny.add_(1.0), 50)
    log(f"launch floor {launch_floor_us:.2f} us per dependent launch")

    # ---------------------------------------------------------------- write sizes
    # the write is latency-bound at 757 tokens: its time over the token count
    sweep = None
    if not args.no_sweep:
        sweep = []
        for n_tok in (32, 128, 757, 1514, 2894, 5788):
            kk = to_dev(normal_bf16(tensor_seed("sweep", n_tok, 1), (n_tok, H, D)))
            vv = to_dev(normal_bf16(tensor_seed("sweep", n_tok, 2), (n_tok, H, D)))
            wsn = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, H, S, D, n_tok), dtype=torch.uint8, device=dev)
            us = graph_us(lambda i: kv.kv_ring_write(ring, kk, vv, 0, 0, tab, workspace=wsn), 20)
            nbytes = n_tok * H * D * (2 * 2 + 2) + 2 * n_tok * H * 4
            sweep.append({"tokens": n_tok, "us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)})
        log("write sweep: " + ", ".join(f"{w['tokens']}: {w['us']:.1f} us ({w['GBps']:.0f} GB/s)" for w in sweep))
        # the ring was overwritten: restore the steady state the later measurements expect
        for c, w in enumerate(sched):
            kv.kv_ring_write(ring, to_dev(normal_bf16(tensor_seed("single_call", c, 1), (N, H, D))),
                             to_dev(normal_bf16(tensor_seed("single_call", c, 2), (N, H, D))),
                             w.start_slot, w.pos0, tab)

    # ---------------------------------------------------------------- fill-up
    # the first chunks of a session attend over a ring that is still filling: attention time
    # over the fill level after each of the 8 writes that fill the ring
    fill = None
    if not args.no_sweep:
        fill = []
        for c in range(8):
            f_c = min((c + 1) * N, S)
            h_c = ((c + 1) * N) % S
            us = graph_us(lambda i: kv.ring_attention(ring, h_c, f_c, q, pos0, tab, scale, out=out, lse=lse,
                                                      workspace=ws_a), 20)
            fill.append({"filled": f_c, "call_us": round(us, 2),
                         "TFLOPs": round(4.0 * N * f_c * D * H / (us * 1e-6) / 1e12, 1)})
        log("fill-up: " + ", ".join(f"{x['filled']}: {x['call_us']:.1f} us" for x in fill))

    # ---------------------------------------------------------------- three-axis positions
    # (frame, row, column) positions: per-token cos/sin rows built on the host once per chunk,
    # the same write / fused call / delta-rotation kernels; a frame reset moves one band
    three = None
    if not args.no_three_axis:
        from workloads import raster_positions
        pos3 = raster_positions(N, 7 * N)
        t0 = time.perf_counter()
        for _ in range(20):
            rows3 = kv.rope_table_3d(pos3, D)
        host_us = (time.perf_counter() - t0) / 20 * 1e6
        tab3 = torch.from_numpy(rows3).to(dev)
        w3_us = graph_us(lambda i: kv.kv_ring_write(ring, k_new, v_new, start, 0, tab3, workspace=ws_w), 50)
        r3_us = graph_us(lambda i: kv.kv_ring_delta_rotate_3d(ring, head, filled, (-5 if i % 2 == 0 else 5, 0, 0),
                                                              workspace=ws_r), 50)

        def step3():
            kv.kv_ring_write_attend(ring, k_new, v_new, start, 0, head, filled, q, 0, tab3, scale,
                                    out=out, lse=lse, workspace=ws_f, stream=stream)
        t_w = time.perf_counter()   # the clock's ramp after the host work above
        while time.perf_counter() - t_w < CLOCK_RAMP_S / 2:
            for _ in range(20):
                step3()
            torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(100):
            step3()
        e1.record(stream)
        torch.cuda.synchronize()
        s3_us = 1000.0 * e0.elapsed_time(e1) / 100
        three = {"step_us": round(s3_us, 2), "write_us": round(w3_us, 2),
                 "write_GBps": round(WRITE_BYTES / (w3_us * 1e-6) / 1e9, 1),
                 "frame_reset_us": round(r3_us, 2),
                 "frame_reset_GBps": round(ROTATE_BYTES / (r3_us * 1e-6) / 1e9, 1),
                 "host_rows_us": round(host_us, 1)}
        log(f"three-axis: step {s3_us:.1f} us, write {w3_us:.1f} us, frame reset {r3_us:.1f} us, "
            f"host rows {host_us:.0f} us per chunk")
        # restore the 1-D ring contents for the measurements below
        for c, w in enumerate(sched):
            kv.kv_ring_write(ring, to_dev(normal_bf16(tensor_seed("single_call", c, 1), (N, H, D))),
                             to_dev(normal_bf16(tensor_seed("single_call", c, 2), (N, H, D))),
                             w.start_slot, w.pos0, tab)

    # ---------------------------------------------------------------- read-time baseline
    # The design the ring replaces: a linear bfloat16 window copied forward by the new tokens,
    # then rotated and quantised whole (one write of S tokens), then the same attention.
    read_time = None
    if not args.no_read_time:
        win = [[to_dev(normal_bf16(tensor_seed("read_time", 0, t), (S, H, D))) for t in (1, 2)],
               [torch.empty((S, H, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]]
        rt_ring = kv.Ring(H, S, D, dev)
        ws_rt = torch.zeros(kv.workspace_bytes(kv.OP_WRITE, H, S, D, S), dtype=torch.uint8, device=dev)
        w_pos0 = pos0 + N - S          # the window ends with the new tokens

        def rt_maintain(i):
            src, dst = win[i % 2], win[(i + 1) % 2]
            kv.kv_window_advance(src[0], dst[0], k_new)        # on torch's current stream
            kv.kv_window_advance(src[1], dst[1], v_new)
            kv.kv_ring_write(rt_ring, dst[0], dst[1], 0, w_pos0, tab, workspace=ws_rt)

        def rt_call(i):
            rt_maintain(i)
            kv.ring_attention(rt_ring, 0, S, q, pos0, tab, scale, out=out, lse=lse, workspace=ws_a,
                              stream=stream)

        for i in range(5):
            rt_call(i)
        # whole calls back to back, timed like the steps above
        e0.record(stream)
        for i in range(reps):
            rt_call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        rt_call_us = 1000.0 * e0.elapsed_time(e1) / reps
        # the maintenance part alone (copies + whole-window write), timed like the write above
        rt_maint_us = graph_us(rt_maintain, 20)
        wt_call_us = gpu_ms * 1000.0      # the timed steps: write + attention, back to back
        read_time = {
            "call_us": round(rt_call_us, 2), "maintenance_us": round(rt_maint_us, 2),
            "write_time_call_us": round(wt_call_us, 2), "write_time_maintenance_us": round(write_gpu_us, 2),
            "maintenance_speedup": round(rt_maint_us / write_gpu_us, 2),
            "call_speedup": round(rt_call_us / wt_call_us, 3),
            "chunk_maintenance_ms": {"read_time": round(240 * rt_maint_us / 1000, 2),
                                     "write_time": round(240 * write_gpu_us / 1000, 2)},
        }
        log(f"read-time call {rt_call_us:.1f} us (maintenance {rt_maint_us:.1f} us) vs write-time "
            f"{wt_call_us:.1f} us (maintenance {write_gpu_us:.1f} us)")
        del win, rt_ring, ws_rt

    # ---------------------------------------------------------------- a 240-call chunk over 60 rings
    chunk = None
    if not args.no_chunk:
        layers, passes = 60, 4
        rings = [ring]
        for _ in range(layers - 1):
            r = kv.Ring(H, S, D, dev)
            r.k.copy_(ring.k)
            r.v.copy_(ring.v)
            r.k_scale.copy_(ring.k_scale)
            r.v_scale.copy_(ring.v_scale)
            rings.append(r)
        gen = torch.Generator(device=dev)
        inputs = []
        for p in range(passes):
            for l in range(layers):
                gen.manual_seed(tensor_seed("full_chunk", p, l))
                inputs.append(tuple(torch.randn((N, H, D), generator=gen, device=dev).to(torch.bfloat16)
                                    for _ in range(3)))

        def run_chunk(st=None):
            for p in range(passes):
                for l in range(layers):
                    kk, vv, qq = inputs[p * layers + l]
                    kv.kv_ring_write_attend(rings[l], kk, vv, start, pos0, head, filled, qq, pos0, tab,
                                            scale, out=out, lse=lse, workspace=ws_f, stream=st)

        run_chunk(stream)
        torch.cuda.synchronize()
        reps_c = 5
        t0 = time.perf_counter()
        for _ in range(reps_c):
            run_chunk(stream)
        torch.cuda.synchronize()
        chunk_ms = (time.perf_counter() - t0) * 1000.0 / reps_c
        # the same 480 library calls captured once in a HIP graph and replayed
        graph_ms = None
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                run_chunk()               # the capture stream is torch's current stream here
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps_c):
                graph.replay()
            torch.cuda.synchronize()
            graph_ms = round((time.perf_counter() - t0) * 1000.0 / reps_c, 3)
            del graph
        chunk = {"calls": passes * layers, "layers": layers, "passes": passes, "ms": round(chunk_ms, 3),
                 "graph_ms": graph_ms}
        log(f"chunk of 240 calls: {chunk_ms:.2f} ms eager, {graph_ms} ms as one graph")
        del inputs, rings

    # ---------------------------------------------------------------- position reset, 60 layers
    # The position-reset workload with outliers: 60 layers' rings hold Student-t (nu = 3) keys and
    # values with 1% of (head, channel) pairs x20, positions 6,212 .. 11,999 (8 writes of 757, the
    # last wrapping); each ring is rotated by delta = -4,000, then 757 queries (N(0,1), positions
    # 7,243 .. 7,999) attend over it.  2.2 GB of rings: every call finds its ring outside the
    # infinity cache (one ring's contents are built once and copied to the other 59).  Timed as
    # the full sequence (60 x (rotate, attend)), then the 60 rotations alone and the 60 attention
    # calls alone; the delta alternates between -4,000 and +4,000 from one repetition to the next
    # so that positions stay inside the rotary table.
    reset = None
    if not args.no_reset:
        from workloads import outlier_channels, student_t_outlier_bf16
        layers = 60
        outl = outlier_channels(tensor_seed("reset", 0, 3), H, D)
        base = kv.Ring(H, S, D, dev)
        rsched = steady_ring_schedule(S, N, 8, 5944)
        for c, w in enumerate(rsched):
            kv.kv_ring_write(base, to_dev(student_t_outlier_bf16(tensor_seed("reset_l0", c, 1), (N, H, D), outl)),
                             to_dev(student_t_outlier_bf16(tensor_seed("reset_l0", c, 2), (N, H, D), outl)),
                             w.start_slot, w.pos0, tab)
        r_head = (rsched[-1].start_slot + N) % S
        rq = to_dev(normal_bf16(tensor_seed("reset_l0", 99, 0), (N, H, D)))
        rings_r = [base]
        for _ in range(layers - 1):
            r = kv.Ring(H, S, D, dev)
            r.k.copy_(base.k), r.v.copy_(base.v), r.k_scale.copy_(base.k_scale), r.v_scale.copy_(base.v_scale)
            rings_r.append(r)
        shift = [0]   # the rings' current position offset (0 or -4,000)
        p_last = rsched[-1].pos0

        def reset_pass(rot=True, att=True):
            d = -4000 if shift[0] == 0 else 4000
            for r in rings_r:
                if rot:
                    kv.kv_ring_delta_rotate(r, r_head, S, d, workspace=ws_r, stream=stream)
                if att:   # queries at the positions the rings hold after this pass's rotation
                    kv.ring_attention(r, r_head, S, rq, p_last + shift[0] + (d if rot else 0), tab, scale,
                                      out=out, lse=lse, workspace=ws_a, stream=stream)
            if rot:
                shift[0] += d

        def timed(rot, att, reps):
            best = None
            for _ in range(reps):
                e0.record(stream)
                reset_pass(rot, att)
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1)
                best = t if best is None else min(best, t)
            return best

        reset_pass(True, True)   # warm-up, then back to the original positions
        reset_pass(True, False)
        torch.cuda.synchronize()
        full_ms = timed(True, True, reps=1)
        rot_ms = timed(True, False, reps=2)
        att_ms = timed(False, True, reps=2)
        reset = {"layers": layers, "ms": round(full_ms, 3),
                 "per_layer_us": round(1000.0 * full_ms / layers, 2),
                 "delta_rotate_us": round(1000.0 * rot_ms / layers, 2),
                 "delta_rotate_GBps": round(ROTATE_BYTES * layers / (rot_ms * 1e-3) / 1e9, 1),
                 "delta_rotate_frac_hbm_peak": round(ROTATE_BYTES * layers / (rot_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 "attention_call_us": round(1000.0 * att_ms / layers, 2),
                 "attention_calls_per_s": round(layers / (att_ms * 1e-3), 1),
                 "data": "Student-t(3) K/V, 1% of (head, channel) pairs x20, N(0,1) queries"}
        log(f"position reset over {layers} rings: {full_ms:.2f} ms ({1000 * full_ms / layers:.1f} us per layer); "
            f"rotations {1000 * rot_ms / layers:.1f} us each ({reset['delta_rotate_GBps']:.0f} GB/s), "
            f"attention {1000 * att_ms / layers:.1f} us per call")
        del rings_r, base

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, sched, k_new, v_new, q, start, pos0, scale)

    value = 1000.0 / ms_per_step
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_s": CLOCK_RAMP_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+fp16",   # E4M3 cache and QK product; fp16 P and widened V in PV
        "data": "synthetic: seeded N(0,1) bfloat16 Q/K/V, ring pre-filled by 8 writes",
        "config": {
            "workload": "one layer call: kv_ring_write of 757 tokens + ring_attention of 757 queries "
                        "over a full 5788-slot FP8 ring, 24 heads x d128 (one GPU's share)",
            "heads": H, "slots": S, "head_dim": D, "new_tokens": N, "queries": N,
        },
        "gpu_ms_per_step": round(gpu_ms, 5),
        "two_call_gpu_ms_per_step": round(sep_ms, 5),
        "attention": {"kernel_us": round(att_us, 2), "call_us": round(call_us, 2),
                      "tflops": round(att_tflops, 1), "frac_fp8_peak": round(att_tflops / FP8_PEAK_TFLOPS, 4),
                      "calls_per_s": round(1e6 / call_us, 1)},
        "write": hbm_entry(write_gpu_us, write_us, WRITE_BYTES, cold["write_us"] if cold else None, copy_gbps),
        "delta_rotate": hbm_entry(rot_gpu_us, rot_us, ROTATE_BYTES, cold["delta_rotate_us"] if cold else None,
                                  copy_gbps),
        "launch_floor_us": round(launch_floor_us, 2),
        "reset_60_layers": reset,
        "hbm_copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "chunk": chunk,
        "cold_cache": cold,
        "write_sweep": sweep,
        "fill_up": fill,
        "three_axis": three,
        "read_time_baseline": read_time,
        # the pages' own figures (four H100, whole model, per diffusion step): context only, not
        # a target for this line's workload
        "context_pages_h100": {"step_ms": {"before": 240.9, "after": 159.3},
                               "cache_maintenance_ms": {"before": 69.7, "after": 6.2},
                               "fp8_cache_saving_ms": 17.0},
        "roofline": {"bound": "mfma", "achieved": round(att_tflops, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(att_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": attention_traffic(), "kernel": ATT_KERNEL, "flop_per_launch": ATT_FLOP},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def hbm_entry(warm_us, issued_us, nbytes, cold_us, copy_gbps):
    """An HBM-bound call: the fraction of HBM peak from its cold-cache GPU time (inputs and outputs
    outside the caches, as in a 60-layer model), with the warm graph-replay time beside it as
    cache-resident throughput."""
    e = {"bytes": nbytes, "cache_resident_us": round(warm_us, 2),
         "cache_resident_GBps": round(nbytes / (warm_us * 1e-6) / 1e9, 1), "issued_us": round(issued_us, 2)}
    if cold_us:
        gbps = nbytes / (cold_us * 1e-6) / 1e9
        e.update({"us": round(cold_us, 2), "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                  "frac_of_copy": round(gbps / copy_gbps, 4) if copy_gbps else None})
    return e


def kernel_sources_hash(read=None) -> str:
    """blake2b of the code (comments, blank lines and trailing blanks dropped) of the sources
    the main attention kernel is compiled from.  `read(name)` returns a source's text."""
    import hashlib
    import re
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "fp8_ring_kv_write_amd", "csrc", name)) as fh:
                return fh.read()
    h = hashlib.blake2b(digest_size=8)
    for f in ("ring_attention.hip", "kvring_common.hpp", "kvring_internal.hpp"):
        for line in read(f).splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def attention_traffic():
    """Counter-measured HBM bytes per launch of the main attention kernel, or None when the
    kernel sources changed since the counters were taken."""
    if ATT_TRAFFIC is None or ATT_TRAFFIC["sources"] != kernel_sources_hash():
        return None
    return ATT_TRAFFIC["bytes"]


def cpu_baseline(np, sched, k_new, v_new, q, start, pos0, scale):
    """The oracle (as it stands) on the same step: write of 757 tokens + attention of 757
    queries over the full ring, 24 heads.  Ring prefill is not timed."""
    import oracle
    from workloads import normal_bf16, tensor_seed
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    table = oracle.rope_table(ROPE_POS, D)
    ring = oracle.OracleRing(H, S, D)
    filled = 0
    for c, w in enumerate(sched):
        oracle.ring_write(ring, normal_bf16(tensor_seed("single_call", c, 1), (N, H, D)),
                          normal_bf16(tensor_seed("single_call", c, 2), (N, H, D)), w.start_slot, w.pos0, table)
        filled = min(filled + N, S)
    head = (sched[-1].start_slot + N) % S
    kb = k_new.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    vb = v_new.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    qb = q.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ring_write(ring, kb, vb, start, pos0, table)
        oracle.ring_attention(ring, head, filled, qb, pos0, table, scale)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 5:
            break
    log(f"cpu oracle: {el / reps:.2f} s per step on {threads} threads")
    # the same step once more with the BLAS pool limited to one thread (one step, bounded)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            oracle.ring_write(ring, kb, vb, start, pos0, table)
            oracle.ring_attention(ring, head, filled, qb, pos0, table, scale)
            single = time.perf_counter() - t1
        log(f"cpu oracle: {single:.2f} s per step on 1 thread")
    except Exception:  # pragma: no cover
        pass
    return {"value": round(reps / el, 4), "unit": "calls/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full steps (write 757 tokens + attention 757x5788, 24 heads x d128), "
                      "numpy float64 attention",
            "single_thread_value": round(1.0 / single, 4) if single else None}


if __name__ == "__main__":
    sys.exit(main())
