#!/usr/bin/env python3
"""Throughput of the low-bit weight-streaming hot path on one MI355X.

One step = one pass of every device entry point at its workload shape, each
on its own freshly drawn weights:

  gemv_w4a16            M=1  K=4096 N=12288        (decode, W4A16 group 128)
  gemv_binplane         M=1  K=4096 N=12288 P=3    (decode, sign planes)
  gemm_smallm_w4a16     M=16 K=4096 N=4096, 12288  (verify block)
  gemm_smallm_binplane  M=16 K=4096 N=4096, 12288  (verify block, P=3)
  lmhead_argmax         M=1  K=4096 N=32768 (trimmed), 248320 (full); M=16 N=32768
  lmhead_verify_greedy  M=16 K=4096 N=248320 (the verify step's head with
                        greedy acceptance of 15 drafted tokens fused)

The metric is weight bytes streamed per second (packed weights + scales +
activations + outputs, the algorithmic bytes of each call) over the whole
step.  Each step reads ~1.3 GB of distinct weights, far more than the 256 MB
last-level cache, so every call streams its weights from HBM.

Also timed, each call on its own but outside the step (so the step and its
`value` keep their definition): the tiny W4A16 mat-vec (M=1 K=256 N=512,
69 KB: launch-bound, so microseconds only); the sa* storage of sign planes (u8 scale
codes per plane and group, one fp16 d per 256-weight super-block) for
decode and verify, P=3, groups of 64 and 128; and W4A16, sign-plane and
sa* blocks of M=32 and M=64 rows (a prefill chunk, the kernels for
16 < M <= 64).

Prints one JSON line.  ``--gpus`` above 1 is refused: this build measures one
GPU's share.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
# The GPU's clocks settle over tens of milliseconds of load, so every timed
# series follows at least this much untimed load of the same work, whatever
# --warmup says (a few warm-up steps alone time part of the ramp).
WARM_S = 0.05
# Copies of a launch-bound call's inputs: it is timed for its latency, not
# for bandwidth, so its inputs are not spread beyond the last-level cache.
LAUNCH_BOUND_COPIES = 64
K = 4096
G = 128


def alg_bytes_linear(kind: str, M: int, N: int, P: int = 0) -> int:
    """Algorithmic bytes of one call: packed weights + scales + X in + Y out."""
    if kind == "w4a16":
        w = N * K // 2 + N * (K // G) * 2
    else:
        w = N * K // 8 * P + P * N * (K // G) * 2
    return w + M * K * 2 + M * N * 2


def alg_bytes_sa(M: int, N: int, P: int, Gs: int) -> int:
    """sa* call: sign planes + one code byte per (plane, row, group) + fp16 d
    per (row, 256 weights) + X in + Y out."""
    return N * K // 8 * P + P * N * (K // Gs) + N * (K // 256) * 2 + M * K * 2 + M * N * 2


def alg_bytes_head(M: int, N: int) -> int:
    """Packed weights + scales + X in + (int32 index, fp32 max) per row out."""
    return N * K // 2 + N * (K // G) * 2 + M * K * 2 + M * 8


def alg_bytes_head_binplane(M: int, N: int, P: int) -> int:
    """Sign planes + fp16 alphas + X in + (int32 index, fp32 max) per row out."""
    return N * K // 8 * P + P * N * (K // G) * 2 + M * K * 2 + M * 8


def build_step(svq, synth, torch):
    """Allocate every call's inputs on the device.

    Returns [(name, bytes, fn, fresh)]: fn runs the call, fresh() allocates
    another copy of the call's inputs (new weights) and returns its runner.
    """
    calls = []
    seed = [100]

    def nxt():
        seed[0] += 1
        return seed[0]

    def lin(kind, M, N, P=0):
        if kind == "w4a16" and M == 1:
            name = f"gemv_w4a16_m1_n{N}"
        elif kind == "w4a16":
            name = f"gemm_smallm_w4a16_m{M}_n{N}"
        elif M == 1:
            name = f"gemv_binplane_p{P}_m1_n{N}"
        else:
            name = f"gemm_smallm_binplane_p{P}_m{M}_n{N}"

        def make():
            if kind == "w4a16":
                blob = synth.device_int4_blob(N, K, nxt())
            else:
                blob = synth.device_binplane_blob(N, K, P, nxt())
            X = synth.device_activations(M, K, nxt()).view(torch.int16)
            Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
            if kind == "w4a16" and M == 1:
                return lambda: svq.gemv_w4a16(blob, X, Y, N, K)
            if kind == "w4a16":
                return lambda: svq.gemm_smallm_w4a16(blob, X, Y, M, N, K)
            if M == 1:
                return lambda: svq.gemv_binplane(blob, X, Y, N, K, P)
            return lambda: svq.gemm_smallm_binplane(blob, X, Y, M, N, K, P)

        calls.append((name, alg_bytes_linear(kind, M, N, P), make(), make))

    heads = {}

    def head(M, N, verify=False):
        def make(blob=None):
            if blob is None:
                blob = synth.device_int4_blob(N, K, nxt())
            X = synth.device_activations(M, K, nxt()).view(torch.int16)
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            mx = torch.empty(M, dtype=torch.float32, device="cuda")
            ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
            if not verify:
                return lambda: svq.lmhead_argmax(blob, X, M, N, K, idx, mx, ws)
            draft = torch.randint(0, N, (M - 1,), dtype=torch.int32, device="cuda")
            tau = torch.empty(1, dtype=torch.int32, device="cuda")
            return lambda: svq.lmhead_verify_greedy(blob, X, M, N, K, draft, idx, mx, tau, ws)

        # The M = 1 and M = 16 heads of one vocabulary share one weight blob.
        if N not in heads:
            heads[N] = synth.device_int4_blob(N, K, nxt())
        name = f"lmhead_verify_greedy_m{M}_n{N}" if verify else f"lmhead_argmax_m{M}_n{N}"
        nbytes = alg_bytes_head(M, N) + (4 * (M - 1) + 4 if verify else 0)
        calls.append((name, nbytes, make(heads[N]), make))

    # Order: the full head (524 MB) sits between uses of anything small, so no
    # call finds its weights in the last-level cache from the previous step.
    head(1, 248320)
    lin("w4a16", 1, 12288)
    lin("binplane", 1, 12288, 3)
    lin("w4a16", 16, 4096)
    lin("w4a16", 16, 12288)
    lin("binplane", 16, 4096, 3)
    lin("binplane", 16, 12288, 3)
    head(1, 32768)
    head(16, 248320, verify=True)  # the verify step: full vocabulary, greedy acceptance fused
    head(16, 32768)                # a block drafter on the trimmed head
    return calls


def build_extra(svq, synth, torch):
    """The calls timed alone, outside the step, in build_step's format: the
    tiny W4A16 mat-vec (M=1 K=256 N=512, launch-bound: microseconds only),
    sa* storage, W4A16 blocks of 32 and 64 rows, and the sign-plane LM head."""
    import numpy as np

    calls = []
    seed = [500]

    def tiny():
        # Drawn on the host (the device generator needs K/128 a multiple of
        # 4) with the workload's distributions, packed by the library.
        case = synth.TINY_W4A16
        codes, scales, x = synth.make_w4a16(case, 0)
        blob0 = torch.from_numpy(svq.pack_int4_grouped(codes, scales)).cuda()
        x0 = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()

        def make():
            blob, xd = blob0.clone(), x0.clone()
            y = torch.empty((1, case.N), dtype=torch.int16, device="cuda")
            return lambda: svq.gemv_w4a16(blob, xd, y, case.N, case.K)

        nbytes = case.N * case.K // 2 + case.N * (case.K // G) * 2 + case.K * 2 + case.N * 2
        calls.append((f"gemv_w4a16_m1_k{case.K}_n{case.N}", nbytes, make(), make))

    def sa(M, N, P, Gs):
        def make():
            seed[0] += 1
            blob = synth.device_sa_blob(N, K, P, Gs, seed[0])
            seed[0] += 1
            X = synth.device_activations(M, K, seed[0]).view(torch.int16)
            Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
            if M == 1:
                return lambda: svq.gemv_sa(blob, X, Y, N, K, P, G=Gs)
            return lambda: svq.gemm_smallm_sa(blob, X, Y, M, N, K, P, G=Gs)

        name = (f"gemv_sa_p{P}_g{Gs}_m1_n{N}" if M == 1 else f"gemm_smallm_sa_p{P}_g{Gs}_m{M}_n{N}")
        calls.append((name, alg_bytes_sa(M, N, P, Gs), make(), make))

    def w4(M, N):
        def make():
            seed[0] += 1
            blob = synth.device_int4_blob(N, K, seed[0])
            seed[0] += 1
            X = synth.device_activations(M, K, seed[0]).view(torch.int16)
            Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
            if M == 1:
                return lambda: svq.gemv_w4a16(blob, X, Y, N, K)
            return lambda: svq.gemm_smallm_w4a16(blob, X, Y, M, N, K)

        name = f"gemv_w4a16_m1_n{N}" if M == 1 else f"gemm_smallm_w4a16_m{M}_n{N}"
        calls.append((name, alg_bytes_linear("w4a16", M, N), make(), make))

    def bpm(M, N, P):
        def make():
            seed[0] += 1
            blob = synth.device_binplane_blob(N, K, P, seed[0])
            seed[0] += 1
            X = synth.device_activations(M, K, seed[0]).view(torch.int16)
            Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
            return lambda: svq.gemm_smallm_binplane(blob, X, Y, M, N, K, P)

        calls.append((f"gemm_smallm_binplane_p{P}_m{M}_n{N}", alg_bytes_linear("binplane", M, N, P), make(), make))

    def bp1(N, P):
        def make():
            seed[0] += 1
            blob = synth.device_binplane_blob(N, K, P, seed[0])
            seed[0] += 1
            X = synth.device_activations(1, K, seed[0]).view(torch.int16)
            Y = torch.empty((1, N), dtype=torch.int16, device="cuda")
            return lambda: svq.gemv_binplane(blob, X, Y, N, K, P)

        calls.append((f"gemv_binplane_p{P}_m1_n{N}", alg_bytes_linear("binplane", 1, N, P), make(), make))

    def bphead(M, N, P):
        def make():
            seed[0] += 1
            blob = synth.device_binplane_blob(N, K, P, seed[0])
            seed[0] += 1
            X = synth.device_activations(M, K, seed[0]).view(torch.int16)
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            mx = torch.empty(M, dtype=torch.float32, device="cuda")
            ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
            return lambda: svq.lmhead_argmax_binplane(blob, X, M, N, K, P, idx, mx, ws)

        calls.append((f"lmhead_argmax_binplane_p{P}_m{M}_n{N}", alg_bytes_head_binplane(M, N, P), make(), make))

    tiny()
    sa(1, 12288, 3, 128)
    sa(16, 4096, 3, 128)
    sa(16, 12288, 3, 128)
    sa(1, 12288, 3, 64)
    sa(16, 12288, 3, 64)
    w4(32, 4096)
    w4(32, 12288)
    w4(64, 4096)
    w4(64, 12288)
    bpm(32, 12288, 3)
    bpm(64, 4096, 3)
    bpm(64, 12288, 3)
    sa(32, 12288, 3, 128)
    sa(64, 12288, 3, 128)
    bphead(1, 32768, 3)
    bphead(16, 32768, 3)
    # M = 1 at N = 4096, so the verify/decode ratio exists for both widths.
    w4(1, 4096)
    bp1(4096, 3)
    return calls


# Launch log: (call, phase, kernel launches) in the order bench.py issues
# them, written with --launch-log so that a profiler's dispatch list can be
# mapped back to calls and phases (every call is one kernel launch; "step"
# entries are whole steps, one launch of every step call each).
LAUNCHES = []


def log_launches(call, phase, n):
    LAUNCHES.append({"call": call, "phase": phase, "launches": int(n)})


def warm_up(torch, run, min_iters=0, min_s=WARM_S):
    """Untimed runs of `run` until at least min_iters of them and min_s
    seconds have passed; returns (seconds, runs)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_iters or time.perf_counter() - t0 < min_s:
        run()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()  # keep the host within a few runs of the GPU
    torch.cuda.synchronize()
    return time.perf_counter() - t0, n


def capture_series(torch, fns, n):
    """One HIP graph of n launches cycling over the runners fns (each runner
    launches on torch's current stream, which is the capture stream inside
    the context), replayed once untimed so its first run is not timed."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fns[i % len(fns)]()
    graph.replay()
    torch.cuda.synchronize()
    return graph


def time_replay(torch, graph, stream, n):
    """Microseconds per launch of one replay of a graph of n launches."""
    begin, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    begin.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return begin.elapsed_time(end) * 1e3 / n


def stream_read_ceiling(svq, torch, nbytes=1 << 30, iters=20, wgs_per_cu=(1, 2, 4), passes=2):
    """GB/s of a plain non-temporal 16-byte streaming read of `nbytes`, cold:
    launches rotate over copies that together hold at least twice the
    last-level cache, so every launch streams from HBM.  The best of the
    given launch widths (workgroups per CU), over `passes` sweeps of them, is
    the ceiling: a short read's rate dips for a while now and then when the
    clocks fall back between the synchronising sweeps, and one sweep can fall
    entirely into such a dip."""
    nbytes = nbytes // 16 * 16
    stride = (nbytes + 255) // 256 * 256
    copies = max(2, -(-2 * LLC_BYTES // stride))
    buf = torch.empty(copies * stride, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(8 * 1024, dtype=torch.int32, device="cuda")
    views = [buf[i * stride: i * stride + nbytes] for i in range(copies)]
    best = 0.0
    stream = torch.cuda.current_stream()
    for w in [w for _ in range(passes) for w in wgs_per_cu]:
        for i in range(3):
            svq.svq_stream_read(views[i % copies], nbytes, sink, w)
        torch.cuda.synchronize()
        runs = [lambda v=v: svq.svq_stream_read(v, nbytes, sink, w) for v in views]
        graph = capture_series(torch, runs, iters)
        _, nw = warm_up(torch, graph.replay, min_s=WARM_S / 5)
        us = time_replay(torch, graph, stream, iters)
        log_launches(f"read_{nbytes}", f"wgs{w}", 3 + iters * (2 + nw))
        del graph
        best = max(best, nbytes / (us * 1e-6) / 1e9)
    del views, buf
    return best


def cpu_baseline(target_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the same step (weight GB/s).

    The sample is every step call cut to its first rows (at least 16), with
    the same K, M and value distributions.  A first pass at 1/64 of the rows
    sizes the sample for about `target_s` seconds of oracle time; when the
    whole step takes less, the whole step is timed several times over.
    """
    import math

    import numpy as np

    import oracle
    from speculative_verify_amd import synth

    shapes = [("w4a16", 1, 12288, 0), ("binplane", 1, 12288, 3), ("w4a16", 16, 4096, 0),
              ("w4a16", 16, 12288, 0), ("binplane", 16, 4096, 3), ("binplane", 16, 12288, 3),
              ("head", 1, 248320, 0), ("head", 1, 32768, 0), ("head", 16, 248320, 0),
              ("head", 16, 32768, 0)]
    rng = np.random.default_rng(7)

    def make(frac, which=shapes):
        jobs = []
        for kind, M, N, P in which:
            n = max(16, int(N * frac) // 16 * 16)
            X = synth.activations(rng, M, K)
            if kind == "binplane":
                signs, alpha = synth.binplane_weights(rng, n, K, P=P)
                jobs.append((lambda s=signs, a=alpha, x=X: oracle.linear_binplane(s, a, x),
                             alg_bytes_linear("binplane", M, n, P)))
            else:
                codes, scales = synth.int4_weights(rng, n, K)
                if kind == "head":
                    jobs.append((lambda c=codes, s=scales, x=X: oracle.argmax_w4a16(c, s, x),
                                 alg_bytes_head(M, n)))
                else:
                    jobs.append((lambda c=codes, s=scales, x=X: oracle.linear_w4a16(c, s, x),
                                 alg_bytes_linear("w4a16", M, n)))
        return jobs

    def run(jobs, reps=1):
        nbytes, secs = 0, 0.0
        for _ in range(reps):
            for fn, b in jobs:
                t0 = time.perf_counter()
                fn()
                secs += time.perf_counter() - t0
                nbytes += b
        return nbytes, secs

    f0 = 1.0 / 64
    _, s0 = run(make(f0))
    frac = f0 * target_s / max(s0, 1e-3)
    reps = 1
    if frac > 1.0:
        reps, frac = min(8, math.ceil(frac)), 1.0
    jobs = make(frac)
    nbytes, secs = run(jobs, reps)
    del jobs
    # One thread, on the mat-vec and verify shapes only (about 3 s).
    threads = oracle.num_threads()
    lin = shapes[:6]
    oracle.set_num_threads(1)
    try:
        f1 = 1.0 / 512
        _, s1 = run(make(f1, lin))
        f1 = min(1.0, f1 * 3.0 / max(s1, 1e-3))
        b1, t1 = run(make(f1, lin))
    finally:
        oracle.set_num_threads(threads)
    return {
        "value": round(nbytes / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"each step call on its first {frac:.2%} of output rows (at least 16), same K, M "
                   f"and value distributions, timed {reps}x: {nbytes / 1e6:.1f} MB of weights in "
                   f"{secs:.1f} s of oracle time"),
        "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "sample": (f"the W4A16 and P3 mat-vec and M=16 verify calls on their first "
                                     f"{f1:.2%} of output rows: {b1 / 1e6:.1f} MB in {t1:.1f} s")},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # Untimed steps before the timed ones; at least WARM_S seconds of steps
    # run in any case.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--launch-log", default=None,
                    help="write the (call, phase, launches) sequence to this JSON file (for profiler summaries)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported "
              "(the path has no collectives; see the sharding notes in the design document).",
              file=sys.stderr)
        return 2

    import torch

    import speculative_verify_amd as svq
    from speculative_verify_amd import synth

    torch.cuda.set_device(0)
    svq.load()
    calls = build_step(svq, synth, torch)
    extra = build_extra(svq, synth, torch)
    step_bytes = sum(c[1] for c in calls)
    torch.cuda.synchronize()

    def one_step():
        for c in calls:
            c[2]()

    warm_step_s, warm_steps = warm_up(torch, one_step, min_iters=args.warmup)
    log_launches("step", "warm", warm_steps)

    # The step throughput: K steps back to back, no events between calls.
    stream = torch.cuda.current_stream()
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(args.steps):
        for c in calls:
            c[2]()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = t_begin.elapsed_time(t_end) / args.steps
    log_launches("step", "timed", args.steps)

    # Per-call durations, each call on its own: K launches back to back,
    # rotating over copies of the call's inputs that together hold at least
    # twice the 256 MB last-level cache, so every launch streams its weights
    # from HBM (the method of the streaming-read ceiling below).  The K
    # launches are captured once into a HIP graph and the graph is replayed
    # between one pair of events: issued one by one from Python, a call's
    # host path (argument marshalling, the runtime's launch) can take longer
    # than a small kernel runs, and the series would time the host.
    kernels = {}
    launch_bound = {c[0] for c in extra if c[0].startswith("gemv_w4a16_m1_k256")}
    for name, nbytes, fn, fresh in calls + extra:
        copies = max(2, -(-2 * LLC_BYTES // nbytes))
        if name in launch_bound:
            copies = LAUNCH_BOUND_COPIES
        rot = [fn] + [fresh() for _ in range(copies - 1)]
        for f in rot[:3]:
            f()
        torch.cuda.synchronize()
        graph = capture_series(torch, rot, args.steps)
        _, nw = warm_up(torch, graph.replay)
        log_launches(name, "warm", len(rot[:3]) + args.steps * (1 + nw))
        # Five timed replays; the median is reported (one alone varies by a
        # few percent from run to run).
        us = sorted(time_replay(torch, graph, stream, args.steps) for _ in range(5))[2]
        log_launches(name, "timed", 5 * args.steps)
        del graph, rot
        # Hot: the same launches on one copy of the inputs, which stays in
        # the caches between launches when it fits (a lower bound on the
        # kernel's own latency and arithmetic, not a bandwidth figure).
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = capture_series(torch, [fn], args.steps)
        _, nw = warm_up(torch, graph.replay, min_s=WARM_S / 5)
        hot_us = time_replay(torch, graph, stream, args.steps)
        log_launches(name, "hot", 3 + args.steps * (2 + nw))
        del graph
        gbps = nbytes / (us * 1e-6) / 1e9
        kernels[name] = {"us": round(us, 3), "bytes": nbytes, "GBps": round(gbps, 1),
                         "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "input_copies": copies,
                         "hot_us": round(hot_us, 3)}
    extra_names = {c[0] for c in extra}
    for name in extra_names:
        kernels[name]["in_step"] = False
    for name in launch_bound:
        # Launch-bound: a latency figure; its bytes per second mean nothing.
        kernels[name]["launch_bound"] = True
        for k in ("GBps", "frac_hbm_peak"):
            kernels[name].pop(k, None)
    dom = max((n for n in kernels if n not in extra_names), key=lambda n: kernels[n]["us"])
    dom_us, dom_bytes = kernels[dom]["us"], kernels[dom]["bytes"]
    dom_gbps = kernels[dom]["GBps"]

    def ratio(a, b):
        return round(kernels[a]["us"] / kernels[b]["us"], 3)

    result = {
        "metric": "weight GB/s & % of HBM peak: GEMV M=1, verify GEMM M=16, LM-head+argmax",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": {"steps": warm_steps, "step_s": round(warm_step_s, 4), "per_call_series_s": WARM_S},
        "ms_per_step": round(ms_per_step, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; uniform INT4 codes / Bernoulli sign bits, U(0.005,0.02) bf16 "
                "scales, fp16 plane scales, N(0,1) bf16 activations)",
        "config": {
            "workload": "decode+verify+lmhead step, K=4096, group 128: W4A16 GEMV M1 N12288; "
                        "binary-plane P3 GEMV M1 N12288; W4A16 and P3 verify GEMM M16 N4096/N12288; "
                        "W4A16 LM head + argmax M1 N248320 (full) and M1/M16 N32768 (trimmed); "
                        "verify head M16 N248320 with fused greedy acceptance",
            "step_bytes": step_bytes,
            "frac_hbm_peak": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "launch_us": round(dom_us, 3),
            "alg_bytes": dom_bytes,
            "input_copies": kernels[dom]["input_copies"],
        },
        "kernels": kernels,
        "verify_over_decode_time": {
            "w4a16_n12288": ratio("gemm_smallm_w4a16_m16_n12288", "gemv_w4a16_m1_n12288"),
            "binplane_n12288": ratio("gemm_smallm_binplane_p3_m16_n12288", "gemv_binplane_p3_m1_n12288"),
            "lmhead_n248320": ratio("lmhead_verify_greedy_m16_n248320", "lmhead_argmax_m1_n248320"),
            "sa_p3_g128_n12288": ratio("gemm_smallm_sa_p3_g128_m16_n12288", "gemv_sa_p3_g128_m1_n12288"),
            "sa_p3_g64_n12288": ratio("gemm_smallm_sa_p3_g64_m16_n12288", "gemv_sa_p3_g64_m1_n12288"),
            "binplane_head_p3_n32768": ratio("lmhead_argmax_binplane_p3_m16_n32768",
                                             "lmhead_argmax_binplane_p3_m1_n32768"),
            "w4a16_n4096": ratio("gemm_smallm_w4a16_m16_n4096", "gemv_w4a16_m1_n4096"),
            "binplane_n4096": ratio("gemm_smallm_binplane_p3_m16_n4096", "gemv_binplane_p3_m1_n4096"),
        },
    }
    traffic = load_traffic(dom)
    if traffic is not None:
        result["roofline"]["traffic"] = traffic
    if not args.no_ceiling:
        # The same-size cold streaming read: what a pure read of each call's
        # bytes achieves with this launch overhead and start-up latency.
        for name, nbytes, _, _ in calls + extra:
            if name in launch_bound:
                continue
            ceil = stream_read_ceiling(svq, torch, nbytes)
            kernels[name]["ceiling_GBps"] = round(ceil, 1)
            kernels[name]["frac_of_ceiling"] = round(kernels[name]["GBps"] / ceil, 4)
        result["stream_read_ceiling_GBps"] = round(stream_read_ceiling(svq, torch, wgs_per_cu=(1,)), 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    if args.launch_log:
        with open(args.launch_log, "w") as f:
            json.dump({"steps": args.steps, "step_calls": [c[0] for c in calls], "launches": LAUNCHES}, f, indent=0)
    print(json.dumps(result), flush=True)
    return 0


def load_traffic(kernel_name: str):
    """HBM bytes per launch of `kernel_name` from the committed counter summary,
    or None when the kernel source changed after the counters were taken."""
    from speculative_verify_amd.build import device_source_digest
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("device_source_sha256") != device_source_digest():
        return None
    return t.get("per_launch_bytes", {}).get(kernel_name)


if __name__ == "__main__":
    sys.exit(main())
