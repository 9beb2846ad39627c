"""Benchmark: selective-scan forward throughput on one MI355X.

A step is one forward selective scan (all of: staging, softplus, ZOH
discretization, recurrence, readout, D skip, SiLU gate, final state) over the
Mamba-1.4B-shaped layer workload: batch 4, d_inner 4096, d_state 16, L 8192,
bf16 io, fp32 state, gated, final state returned.  Inputs are synthetic
(seeded), resident in HBM before timing starts.

Prints one JSON line with the throughput in Gtok*ch/s, the algorithmic HBM
bandwidth, a roofline record for the scan kernel and the fp64 oracle's
throughput on the host cores (CPU baseline, on a bounded sample).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan fwd Gtok·ch/s and achieved HBM GB/s (% of peak), 1.4B shape"
HBM_PEAK_GBPS = 8000.0
# ALU peak: MI355X's published fp32 vector rate, 157.3 TFLOP/s, is 256 CUs x 2.4 GHz x 128 FMA
# lanes per CU per clock: 78.6 T lane-op issue slots/s (an FMA, multiply or add fills one slot).
# A transcendental (v_exp_f32, v_log_f32, v_rcp_f32) issues at a quarter of that rate
# (measured ~31 lane-ops per CU per clock against ~90 for VGPR-only FMAs at two waves per SIMD),
# so it counts as 4 slots.  Counts below are the method's own arithmetic per unit of work, not
# what the kernels execute (the accurate expm1 of the decay, conversions, address and
# cross-lane work are implementation overhead).
VALU_SLOTS_PEAK = 256 * 2.4e9 * 128
TRANS = 4.0
# forward, per (token, channel, state): Delta*A, exp, u/A, *B, h + s, the update FMA, the
# readout FMA; Euler: Delta*A, exp, B*(Delta u), the update FMA, the readout FMA
SLOTS_PER_TCN = 6.0 + TRANS
SLOTS_PER_TCN_EULER = 4.0 + TRANS
# per (token, channel): softplus (exp + log + 3 ops), the SiLU gate (exp + rcp + 3 ops + the
# multiply) and the D skip; ungated: softplus and the D skip
SLOTS_PER_TC_GATED = (2 * TRANS + 3) + (2 * TRANS + 4) + 1
SLOTS_PER_TC_UNGATED = (2 * TRANS + 3) + 1
CSRC = os.path.join(ROOT, "selective_state_space_55_amd", "csrc")
# committed rocprofv3 traffic summaries and the device sources (kernel file + io helpers) they were taken on
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "scan_fwd_mamba1.4b_traffic.txt")
# HBM-traffic summaries of the forward per workload index (all kernels of one call, default plan)
PROFILE_TRAFFIC_FWD = {2: PROFILE_TRAFFIC, 3: os.path.join(ROOT, "profiles", "scan_fwd_million_traffic.txt")}
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("scan_fwd.hip", "scan_fwd_h2.h", "io.h")]
PROFILE_TRAFFIC_STEP = os.path.join(ROOT, "profiles", "scan_step_decode2.8b_traffic.txt")
KERNEL_SOURCES_STEP = [os.path.join(CSRC, f) for f in ("scan_step.hip", "io.h")]
PROFILE_TRAFFIC_CONV = os.path.join(ROOT, "profiles", "conv1d_mamba1.4b_traffic.txt")
KERNEL_SOURCES_CONV = [os.path.join(CSRC, f) for f in ("conv1d.hip", "io.h")]
PROFILE_TRAFFIC_SSD = os.path.join(ROOT, "profiles", "ssd_fwd_layer_traffic.txt")
PROFILE_TRAFFIC_CONV_FUSED = os.path.join(ROOT, "profiles", "scan_fwd_conv_mamba1.4b_traffic.txt")
KERNEL_SOURCES_SSD = [os.path.join(CSRC, f) for f in ("ssd_fwd.hip", "io.h")]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in (sources or KERNEL_SOURCES):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(nbytes_alg: float, profile: str = PROFILE_TRAFFIC, sources=None):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    if it was taken on the current kernel source; else None."""
    if not os.path.exists(profile):
        return None
    kv = {}
    for line in open(profile):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


CACHE_BYTES = 256 << 20   # MI355X Infinity Cache


def flushed_launch_ms(launch, stream, reps: int) -> float:
    """Median device time of `launch` when a 1 GiB scratch write on the same stream precedes each
    launch, so the inputs come from HBM rather than the 256 MB Infinity Cache."""
    import torch

    scratch = torch.empty(1 << 28, dtype=torch.float32, device=stream.device)
    ts = []
    for r in range(reps):
        scratch.fill_(float(r))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(r)
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    vals = sorted(e0.elapsed_time(e1) for e0, e1 in ts)
    del scratch
    return vals[len(vals) // 2]


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def bench_step(args, c) -> int:
    """Decode-step workload: `steps` chained single-token updates of a (batch, dim, N)
    fp32 state, fresh seeded inputs per step (a pool of 64 distinct steps, resident)."""
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import step_initial, step_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    init = step_initial(c)
    pool = 64
    ins = [step_inputs(c, k) for k in range(pool)]
    x = torch.stack([i["x"] for i in ins]).to(dev)
    dt = torch.stack([i["dt"] for i in ins]).to(dev)
    z = torch.stack([i["z"] for i in ins]).to(dev)
    Bm = torch.stack([i["B"] for i in ins]).to(dev)
    Cm = torch.stack([i["C"] for i in ins]).to(dev)
    st = init["state"].to(dev)
    A, D, bias = init["A_log"].to(dev), init["D"].to(dev), init["dt_bias"].to(dev)
    y = torch.empty((c.batch, c.dim), dtype=x.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(k, state, strm=None):
        j = k % pool
        mscan.scan_step(state, x[j], dt[j], A, Bm[j], Cm[j], D=D, z=z[j], dt_bias=bias, out=y, stream=strm,
                        discretization=args.discretization)

    # A decode loop is launch-bound from Python, so the K chained steps are
    # captured once in a HIP graph and replayed; the replay is checked against
    # the same K steps launched one by one (bit-exact: same kernels, same order).
    st0 = st.clone()
    for k in range(args.warmup):
        step(k, st, stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(args.steps):
            step(k, st)          # the capture stream is the current stream here
    st.copy_(st0)
    graph.replay()
    st_eager = st0.clone()
    for k in range(args.steps):
        step(k, st_eager, stream)
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(st, st_eager))
    if not graph_ok:
        print("bench.py: graph replay differs from eager steps", file=sys.stderr)
        return 1
    for _ in range(max(1, args.warmup // max(1, args.steps))):
        graph.replay()
    torch.cuda.synchronize()
    st_pre = st.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    dev_ms = e0.elapsed_time(e1) / args.steps
    # the timed replay too must equal eager steps from the state it started from
    for k in range(args.steps):
        step(k, st_pre, stream)
    torch.cuda.synchronize()
    graph_ok = graph_ok and bool(torch.equal(st, st_pre))
    if not graph_ok:
        print("bench.py: timed graph replay differs from eager steps", file=sys.stderr)
        return 1
    bd = c.batch * c.dim
    alg = c.algorithmic_bytes()
    # cold-cache leg: the 84 MB state fits the Infinity Cache, so each of these steps follows a
    # 1 GiB scratch write (the steps stay chained: each reads the state the previous one wrote)
    flushed_ms = flushed_launch_ms(lambda r: step(r, st, stream), stream, max(11, min(args.steps, 50)))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        ref = init["state"].double().numpy()
        A_h, D_h, bias_h = init["A_log"], init["D"], init["dt_bias"]
        c0 = time.perf_counter()
        nst = 0
        # chained steps over the whole state until ~15 s of host time (all 1024 if they fit)
        while nst < c.steps and (nst < 4 or time.perf_counter() - c0 < 15.0):
            i = ins[nst % pool]
            _, ref = oracle.scan_step(ref, i["x"], i["dt"], A_h, i["B"], i["C"], D=D_h, z=i["z"], dt_bias=bias_h,
                                      discretization=args.discretization, nthreads=cores)
            nst += 1
        cs = time.perf_counter() - c0
        cpu = {"value": round(bd * nst / cs / 1e9, 6), "unit": "G(batch*channel) updates/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{nst} chained steps of the whole workload ({c.batch} x {c.dim} x {c.dstate} fp64 state), "
                         f"{cs:.2f} s wall incl. fp64 widening of each step's inputs"}
    out = {
        "metric": "selective-scan decode step throughput (state updates per second)",
        "value": round(bd / (dev_ms * 1e-3) / 1e9, 3),
        "unit": "G(batch*channel) updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "device_ms_per_step": round(dev_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{c.name}: batch {c.batch}, d_inner {c.dim}, d_state {c.dstate}, fp32 state, "
                               f"{c.io} io, gated, chained steps replayed from one HIP graph",
                   "batch": c.batch, "d_inner": c.dim, "d_state": c.dstate, "graph_matches_eager": graph_ok},
        "roofline": {"bound": "hbm", "achieved": round(alg / (dev_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(alg / (dev_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": (read_traffic(alg, PROFILE_TRAFFIC_STEP, KERNEL_SOURCES_STEP)
                                 if args.discretization == "zoh" else None)},
        "flushed": {"device_ms_per_step": round(flushed_ms, 5),
                    "GBps": round(alg / (flushed_ms * 1e-3) / 1e9, 1),
                    "frac_of_8TBps": round(alg / (flushed_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "note": "eager steps, each after a 1 GiB scratch write (cold Infinity Cache); "
                            "the headline figure above is warm, replayed from a HIP graph"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# algorithmic slots of the backward pass: per (token, channel, state) one forward recompute
# (SLOTS_PER_TCN) and the gradient terms (lam, Abar lam, dDelta, du, dB, dC and dA's two running
# sums: 9); per (token, channel) softplus and its derivative (a sigmoid: exp + rcp + 2), SiLU and
# its derivative (exp + rcp + 5) and the D terms (2); ungated: softplus and its derivative, D
SLOTS_BWD_PER_TCN = SLOTS_PER_TCN + 9.0
SLOTS_BWD_PER_TC_GATED = (2 * TRANS + 3) + (2 * TRANS + 2) + (2 * TRANS + 5) + 2
SLOTS_BWD_PER_TC_UNGATED = (2 * TRANS + 3) + (2 * TRANS + 2) + 2


PROFILE_TRAFFIC_BWD = os.path.join(ROOT, "profiles", "scan_bwd_mamba1.4b_traffic.txt")
KERNEL_SOURCES_BWD = [os.path.join(CSRC, f) for f in ("scan_bwd.hip", "io.h")]


def BWD_BYTES_PER_TC(c) -> int:
    """Algorithmic HBM bytes of the backward per (token, channel): read u, delta, dy (and z), write
    du, ddelta (and dz); B, C, dB, dC and the parameters are per (token, state) or smaller."""
    e = c.io_bytes()
    return e * (5 + (2 if c.gated else 0))


def bench_bwd(args, c) -> int:
    """Backward pass of a forward workload: gradients of all inputs from a seeded dy."""
    import numpy as np
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import backward_inputs, forward_inputs, max_rel_err

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = forward_inputs(c)
    b, d, n, L = c.batch, c.dim, c.dstate, c.seqlen
    dy, _ = backward_inputs(b, d, n, L, c.io, seed=0)
    a = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    dyd = dy.to(dev)
    io = mscan.BF16 if c.io == "bf16" else mscan.F32
    ws = torch.empty(mscan.bwd_workspace_size(b, d, n, L, io) + 256, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return mscan.scan_bwd(a["u"], a["delta"], a["A_log"], a["B"], a["C"], dyd, D=a["D"], z=a["z"],
                              delta_bias=a["delta_bias"], workspace=ws, stream=stream,
                              discretization=args.discretization)

    for _ in range(args.warmup):
        g = step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    w0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        g = step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    launch_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    tc = b * d * L
    slots = tc * n * SLOTS_BWD_PER_TCN + tc * (SLOTS_BWD_PER_TC_GATED if c.gated else SLOTS_BWD_PER_TC_UNGATED)
    achieved = slots / (launch_ms * 1e-3) / 1e12

    parity = None
    if not args.no_parity:
        import oracle

        # sampled check: batch row 0, channels 0..63 (dB, dC need every channel of the row,
        # so they are compared on a 64-channel problem run on both sides)
        sub = {k: (v[:1, :64] if (v is not None and k in ("u", "delta", "z")) else
                   (v[:1] if (v is not None and k in ("B", "C")) else
                    (v[:64] if (v is not None and k in ("A_log", "D", "delta_bias")) else v)))
               for k, v in inp.items()}
        dys = dy[:1, :64].contiguous()
        gs = mscan.scan_bwd(*(t.contiguous().to(dev) for t in (sub["u"], sub["delta"], sub["A_log"], sub["B"],
                                                               sub["C"], dys)),
                            D=sub["D"].to(dev), z=None if sub["z"] is None else sub["z"].contiguous().to(dev),
                            delta_bias=sub["delta_bias"].to(dev), discretization=args.discretization)
        r = oracle.scan_bwd(sub["u"], sub["delta"], sub["A_log"], sub["B"], sub["C"], dys, D=sub["D"], z=sub["z"],
                            delta_bias=sub["delta_bias"], discretization=args.discretization)
        parity = {k: max_rel_err(gs[k].float().cpu(), r[k]) for k in ("du", "ddelta", "dA_log", "dB", "dC", "dD")}
        parity["tol"] = c.tol
        parity["sample"] = "batch row 0, channels 0-63, full length"

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        # bounded sample: batch row 0, the first channels, full length (~1e9 (token, channel, state))
        nch = int(min(d, max(1, 1e9 // (L * n))))
        sub = {k: (v[:1, :nch] if (v is not None and k in ("u", "delta", "z")) else
                   (v[:1] if (v is not None and k in ("B", "C")) else
                    (v[:nch] if (v is not None and k in ("A_log", "D", "delta_bias")) else v)))
               for k, v in inp.items()}
        c0 = time.perf_counter()
        oracle.scan_bwd(sub["u"], sub["delta"], sub["A_log"], sub["B"], sub["C"], dy[:1, :nch], D=sub["D"],
                        z=sub["z"], delta_bias=sub["delta_bias"], discretization=args.discretization, nthreads=cores)
        cs = time.perf_counter() - c0
        cpu = {"value": round(nch * L / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"batch row 0 x {nch} channels x {L} tokens x {n} states, all gradients, fp64, "
                         f"{cs:.2f} s wall incl. fp64 widening of inputs"}

    out = {
        "metric": "selective-scan backward Gtok·ch/s (all input gradients)",
        "value": round(tc / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{c.name} selective-scan backward: batch {b}, d_inner {d}, d_state {n}, L {L}, "
                               f"{c.io} io, fp32 state, {'gated' if c.gated else 'ungated'}, {args.discretization}",
                   "batch": b, "d_inner": d, "d_state": n, "seqlen": L},
        "kernel_ms": round(launch_ms, 4),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_SLOTS_PEAK / 1e12, 3),
                     "unit": "T fp32 lane-op slots/s", "frac": round(achieved / (VALU_SLOTS_PEAK / 1e12), 4),
                     "traffic": read_traffic(tc * BWD_BYTES_PER_TC(c), PROFILE_TRAFFIC_BWD, KERNEL_SOURCES_BWD)},
        "hbm": {"algorithmic_bytes": tc * BWD_BYTES_PER_TC(c),
                "GBps": round(tc * BWD_BYTES_PER_TC(c) / (launch_ms * 1e-3) / 1e9, 1),
                "frac_of_8TBps": round(tc * BWD_BYTES_PER_TC(c) / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": cpu,
        "parity_sampled": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


def _graph_timing(args, step, u, stream):
    """Times K launches replayed from one HIP graph: (ms per launch, wall s), or None if the
    replayed output u differs from the eager launch's."""
    import torch

    # One launch is shorter than the Python call that makes it, so the K steps
    # are captured once in a HIP graph and replayed (as for decoding); the
    # replayed output must equal an eager launch's bit for bit.
    step(stream)
    torch.cuda.synchronize()
    u_eager = u.clone()
    u.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()               # the capture stream is the current stream here
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(u, u_eager):
        print("bench.py: graph replay differs from the eager launch", file=sys.stderr)
        return None
    for _ in range(max(1, args.warmup // max(1, args.steps))):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    launch_ms = e0.elapsed_time(e1) / args.steps
    return launch_ms, wall


def bench_conv(args, c) -> int:
    """Causal depthwise conv1d (K = 4) + SiLU over the forward config's (batch, d_inner, L)
    input, the step in front of the scan in the Mamba block: a pure HBM stream."""
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import conv_inputs, max_rel_err

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    b, d, L, K = c.batch, c.dim, c.seqlen, 4
    x, w, bias, _ = conv_inputs(b, d, L, K, c.io, seed=0)
    xd, wd, bd = x.to(dev), w.to(dev), bias.to(dev)
    u = torch.empty_like(xd)
    stream = torch.cuda.current_stream(dev)

    def step(strm=None):
        mscan.conv1d_fwd(xd, wd, bd, out=u, stream=strm)

    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    if args.no_graph:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        w0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        launch_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    else:
        r = _graph_timing(args, step, u, stream)
        if r is None:
            return 1
        launch_ms, wall = r
    ms_per_step = wall * 1e3 / args.steps
    tc = b * d * L
    alg_bytes = 2 * tc * x.element_size() + d * (K + 1) * 4   # read x, write u, weights + bias
    gbps = alg_bytes / (launch_ms * 1e-3) / 1e9
    traffic = read_traffic(alg_bytes, PROFILE_TRAFFIC_CONV, KERNEL_SOURCES_CONV)

    parity = None
    if not args.no_parity:
        import oracle

        rows = [(0, 0), (b // 2, d // 2 + 1), (b - 1, d - 1)]
        err = 0.0
        for bb, dd in rows:
            ur = oracle.conv1d_fwd(x[bb:bb + 1, dd:dd + 1], w[dd:dd + 1], bias[dd:dd + 1])
            err = max(err, max_rel_err(u[bb:bb + 1, dd:dd + 1].float().cpu(), ur))
        parity = {"rows": rows, "u_max_rel": err, "tol": 1e-2 if c.io == "bf16" else 1e-5}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        nrow = min(b * d, max(1, int(5e8 // L)))
        xs = x.view(b * d, L)[:nrow].view(1, nrow, L)
        c0 = time.perf_counter()
        oracle.conv1d_fwd(xs, w.repeat((nrow + d - 1) // d, 1)[:nrow], bias.repeat((nrow + d - 1) // d)[:nrow],
                          nthreads=cores)
        cs = time.perf_counter() - c0
        cpu = {"value": round(nrow * L / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"{nrow} of {b * d} (batch, channel) rows x {L} tokens, K {K}, fp64, {cs:.2f} s wall "
                         "incl. fp64 widening of inputs"}

    out = {
        "metric": "causal conv1d + SiLU Gtok·ch/s and achieved HBM GB/s",
        "value": round(tc / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{c.name} causal depthwise conv1d + SiLU: batch {b}, d_inner {d}, L {L}, K {K}, "
                               f"{c.io} io, bias, "
                               + ("eager launches" if args.no_graph else "launches replayed from one HIP graph"),
                   "batch": b, "d_inner": d, "seqlen": L, "K": K},
        "kernel_ms": round(launch_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "parity_sampled": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


# causal conv1d (K = 4) + SiLU per (token, channel): 4 FMAs, exp, add, rcp, multiply
SLOTS_PER_TC_CONV = 6.0 + 2 * TRANS


def bench_conv_fused(args, c) -> int:
    """The causal conv1d (K = 4) + SiLU fused into the forward scan's load stage, over the forward
    config (the scan input u never goes through HBM); the same work as two separate launches
    (conv1d, then the scan) is timed alongside for comparison."""
    import numpy as np
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import conv_inputs, forward_inputs, max_rel_err

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = forward_inputs(c)
    _, w, cbias, _ = conv_inputs(c.batch, c.dim, c.seqlen, 4, c.io, seed=0)
    a = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    wd, cbd = w.to(dev), cbias.to(dev)
    b, d, n, L = c.batch, c.dim, c.dstate, c.seqlen
    io = mscan.BF16 if c.io == "bf16" else mscan.F32
    ws_bytes = mscan.fwd_workspace_size(b, d, n, L, io)
    ws = torch.empty(max(ws_bytes, 1) + 256, dtype=torch.uint8, device=dev)
    y = torch.empty((b, d, L), dtype=a["u"].dtype, device=dev)
    fs = torch.empty((b, d, n), dtype=torch.float32, device=dev)
    u = torch.empty_like(a["u"])
    stream = torch.cuda.current_stream(dev)

    def fused():
        mscan.scan_fwd_conv(a["u"], wd, a["delta"], a["A_log"], a["B"], a["C"], D=a["D"], z=a["z"],
                            delta_bias=a["delta_bias"], conv_bias=cbd, out=y, final_state=fs,
                            return_final_state=True, workspace=ws, stream=stream,
                            discretization=args.discretization)

    def separate():
        mscan.conv1d_fwd(a["u"], wd, cbd, out=u, stream=stream)
        mscan.scan_fwd(u, a["delta"], a["A_log"], a["B"], a["C"], D=a["D"], z=a["z"], delta_bias=a["delta_bias"],
                       out=y, final_state=fs, return_final_state=True, workspace=ws, stream=stream,
                       discretization=args.discretization)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        w0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps, wall * 1e3 / args.steps

    sep_ms, _ = timed(separate)
    y_sep = y.clone()
    fs_sep = fs.clone()
    launch_ms, ms_per_step = timed(fused)
    identical = bool(torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                                 y_sep.view(torch.int16) if y.dtype == torch.bfloat16 else y_sep)
                     and torch.equal(fs, fs_sep))

    tc = b * d * L
    per_tcn = SLOTS_PER_TCN if args.discretization == "zoh" else SLOTS_PER_TCN_EULER
    slots = tc * n * per_tcn + tc * ((SLOTS_PER_TC_GATED if c.gated else SLOTS_PER_TC_UNGATED) + SLOTS_PER_TC_CONV)
    achieved = slots / (launch_ms * 1e-3) / 1e12
    peak = VALU_SLOTS_PEAK / 1e12
    alg_bytes = c.algorithmic_bytes() + d * 5 * 4   # x in place of u, plus taps and conv bias

    def oracle_rows(rows):
        import oracle

        ys, fss = [], []
        for r in rows:
            bb, dd = divmod(r, d)
            u64 = oracle.conv1d_fwd(inp["u"][bb:bb + 1, dd:dd + 1], w[dd:dd + 1], cbias[dd:dd + 1])
            u_io = torch.from_numpy(np.asarray(u64, dtype=np.float32)).to(inp["u"].dtype)
            yr, fr = oracle.scan_fwd(u_io, inp["delta"][bb:bb + 1, dd:dd + 1], inp["A_log"][dd:dd + 1],
                                     inp["B"][bb:bb + 1], inp["C"][bb:bb + 1],
                                     D=None if inp["D"] is None else inp["D"][dd:dd + 1],
                                     z=None if inp["z"] is None else inp["z"][bb:bb + 1, dd:dd + 1],
                                     delta_bias=None if inp["delta_bias"] is None else inp["delta_bias"][dd:dd + 1],
                                     discretization=args.discretization)
            ys.append(yr[0, 0])
            fss.append(fr[0, 0])
        return np.stack(ys), np.stack(fss)

    parity = None
    if not args.no_parity:
        rows = [0, d // 2 + 7, (b - 1) * d + d - 1]
        yr, fr = oracle_rows(rows)
        parity = {"rows": rows, "y_max_rel": max_rel_err(y.view(b * d, L)[rows].cpu(), yr),
                  "final_state_max_rel": max_rel_err(fs.view(b * d, n)[rows].cpu(), fr), "tol": c.tol}

    cpu = None
    if not args.no_cpu_baseline:
        nrow = 512
        c0 = time.perf_counter()
        oracle_rows(list(range(nrow)))
        cs = time.perf_counter() - c0
        cpu = {"value": round(nrow * L / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": 1, "kind": "oracle",
               "sample": f"{nrow} of {b * d} (batch, channel) rows x {L} tokens: oracle conv1d, u rounded to "
                         f"{c.io}, oracle scan, fp64, one row at a time, {cs:.2f} s wall"}

    out = {
        "metric": "causal conv1d + SiLU + selective-scan fwd Gtok·ch/s (conv fused into the scan)",
        "value": round(tc / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{c.name} conv1d (K 4, bias) + SiLU + selective scan: batch {b}, d_inner {d}, "
                               f"d_state {n}, L {L}, {c.io} io, fp32 state, "
                               + ("gated" if c.gated else "ungated") + f", {args.discretization}",
                   "batch": b, "d_inner": d, "d_state": n, "seqlen": L},
        "kernel_ms": round(launch_ms, 4),
        "separate_ms": round(sep_ms, 4),
        "identical_to_separate": identical,
        "hbm_gbps": round(alg_bytes / (launch_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(peak, 3),
                     "unit": "T fp32 lane-op slots/s", "frac": round(achieved / peak, 4),
                     "traffic": (read_traffic(alg_bytes, PROFILE_TRAFFIC_CONV_FUSED)
                                 if args.discretization == "zoh" else None)},
        "cpu_baseline": cpu,
        "parity_sampled": parity,
    }
    print(json.dumps(out), flush=True)
    return 0 if identical else 1


def bench_varlen(args, c) -> int:
    """Variable-length batch over the forward config's channels and total tokens: batch x L tokens
    per channel split into a seeded mix of sequence lengths (uniform 64..2048, the last one
    trimmed), packed along time, each sequence from its own initial state."""
    import numpy as np
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import forward_inputs, max_rel_err

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    total = c.batch * c.seqlen
    rng = np.random.default_rng(1234)
    lens = []
    if args.varlen_lens:
        lens = [int(x) for x in args.varlen_lens.split(",")]
        total = sum(lens)
    while sum(lens) < total:
        lens.append(int(min(rng.integers(64, 2049), total - sum(lens))))
    nseq = len(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    inp = forward_inputs(batch=1, dim=c.dim, dstate=c.dstate, seqlen=total, io=c.io, gated=c.gated, seed=0)
    a = {k: (None if v is None else (v[0] if v.dim() == 3 else v).to(dev)) for k, v in inp.items()
         if k != "initial_state"}
    h0 = (torch.randn(nseq, c.dim, c.dstate, generator=torch.Generator().manual_seed(3)) * 0.1).to(dev)
    cud = cu.to(dev)
    y = torch.empty_like(a["u"])
    fs = torch.empty(nseq, c.dim, c.dstate, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mscan.scan_fwd_varlen(a["u"], a["delta"], a["A_log"], a["B"], a["C"], cud, D=a["D"], z=a["z"],
                              delta_bias=a["delta_bias"], initial_states=h0, out=y, final_states=fs,
                              return_final_states=True, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    w0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    launch_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    tc = total * c.dim
    slots = tc * c.dstate * SLOTS_PER_TCN + tc * (SLOTS_PER_TC_GATED if c.gated else SLOTS_PER_TC_UNGATED)
    achieved = slots / (launch_ms * 1e-3) / 1e12

    parity = None
    if not args.no_parity:
        import oracle

        chans = [0, c.dim // 2 + 3, c.dim - 1]
        host = {k: (None if v is None else v.cpu()) for k, v in a.items()}
        yr, fr = oracle.scan_fwd_varlen(host["u"][chans], host["delta"][chans], host["A_log"][chans], host["B"],
                                        host["C"], cu.numpy(), D=host["D"][chans],
                                        z=None if host["z"] is None else host["z"][chans],
                                        delta_bias=host["delta_bias"][chans], initial_states=h0.cpu()[:, chans])
        parity = {"channels": chans, "y_max_rel": max_rel_err(y.cpu()[chans], yr),
                  "final_states_max_rel": max_rel_err(fs.cpu()[:, chans], fr), "tol": c.tol}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        # bounded sample: the first channels, every sequence, full length (~2e9 updates)
        nch = int(min(c.dim, max(1, 2e9 // (total * c.dstate))))
        host = {k: (None if v is None else v.cpu()) for k, v in a.items()}
        c0 = time.perf_counter()
        oracle.scan_fwd_varlen(host["u"][:nch], host["delta"][:nch], host["A_log"][:nch], host["B"], host["C"],
                               cu.numpy(), D=host["D"][:nch], z=None if host["z"] is None else host["z"][:nch],
                               delta_bias=host["delta_bias"][:nch], initial_states=h0.cpu()[:, :nch],
                               nthreads=cores)
        cs = time.perf_counter() - c0
        cpu = {"value": round(nch * total / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"{nch} channels x all {nseq} sequences ({total} tokens) x {c.dstate} states, fp64, "
                         f"{cs:.2f} s wall incl. fp64 widening of inputs"}

    out = {
        "metric": "selective-scan fwd over a variable-length batch, Gtok·ch/s",
        "value": round(tc / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{c.name} channels, variable-length batch: {nseq} sequences of "
                               + (f"lengths {args.varlen_lens}" if args.varlen_lens else "64-2048 tokens (seeded uniform)")
                               + f", {total} tokens, d_inner {c.dim}, d_state {c.dstate}, {c.io} io, "
                               f"{'gated' if c.gated else 'ungated'}, per-sequence initial and final states",
                   "nseq": nseq, "total_tokens": total, "d_inner": c.dim, "d_state": c.dstate},
        "kernel_ms": round(launch_ms, 4),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_SLOTS_PEAK / 1e12, 3),
                     "unit": "T fp32 lane-op slots/s", "frac": round(achieved / (VALU_SLOTS_PEAK / 1e12), 4),
                     "traffic": None},
        "cpu_baseline": cpu,
        "parity_sampled": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_ssd(args) -> int:
    """Multi-head SSM with a scalar decay per head (state-space-duality form) on a layer of the same
    width as the 1.4B-shaped forward: batch 4, L 8192, 64 heads of 64 channels (d_inner 4096),
    d_state 128, bf16, D skip, no gate, final state."""
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import max_rel_err, ssd_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    b, L, H, P, N = 4, 8192, 64, 64, 128
    inp = ssd_inputs(b, L, H, P, N, seed=0)
    a = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    y = torch.empty_like(a["x"])
    fs = torch.empty(b, H, P, N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(strm=None):
        mscan.ssd_fwd(a["x"], a["dt"], a["A_log"], a["B"], a["C"], D=a["D"], dt_bias=a["dt_bias"], out=y,
                      final_state=fs, return_final_state=True, stream=strm)

    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    r = _graph_timing(args, step, y, stream)
    if r is None:
        return 1
    launch_ms, wall = r
    ms_per_step = wall * 1e3 / args.steps
    tok_ch = b * L * H * P
    alg_bytes = 2 * tok_ch * 2 + 2 * b * L * N * 2 + b * L * H * 2 + b * H * P * N * 4 + 3 * H * 4
    gbps = alg_bytes / (launch_ms * 1e-3) / 1e9
    # matrix-core work as implemented per (batch, head, 64-token chunk): three 32x32 tiles of
    # B C^T over N, C S (64 x 64 over N), the masked M X (two 32-row tiles over 32 and 64 tokens),
    # the state update (N x 64 over 64 tokens, high and low parts)
    chunks = b * H * ((L + 63) // 64)
    macs = chunks * (3 * 32 * 32 * N + 64 * 64 * N + 32 * 32 * (32 + 64) * 2 + 2 * N * 64 * 64)
    tflops = 2 * macs / (launch_ms * 1e-3) / 1e12

    parity = None
    if not args.no_parity:
        import oracle

        errs = {}
        for bb, hh in [(0, 0), (3, 63)]:
            sub = dict(x=inp["x"][bb:bb + 1, :, hh:hh + 1], dt=inp["dt"][bb:bb + 1, :, hh:hh + 1],
                       A_log=inp["A_log"][hh:hh + 1], B=inp["B"][bb:bb + 1], C=inp["C"][bb:bb + 1],
                       D=inp["D"][hh:hh + 1], dt_bias=inp["dt_bias"][hh:hh + 1])
            yr, fr = oracle.ssd_fwd(**sub)
            errs[f"b{bb}h{hh}"] = {"y": max_rel_err(y[bb:bb + 1, :, hh:hh + 1].cpu(), yr),
                                   "final_state": max_rel_err(fs[bb:bb + 1, hh:hh + 1].cpu(), fr)}
        parity = {"heads": errs, "tol": 1e-2}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        # the whole workload (a few seconds of fp64 work on the host cores)
        c0 = time.perf_counter()
        oracle.ssd_fwd(inp["x"], inp["dt"], inp["A_log"], inp["B"], inp["C"], D=inp["D"], dt_bias=inp["dt_bias"],
                       nthreads=cores)
        cs = time.perf_counter() - c0
        cpu = {"value": round(tok_ch / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"the whole workload: {b} batch rows x {H} heads x {P} channels x {L} tokens x {N} states, "
                         f"fp64, {cs:.2f} s wall incl. fp64 widening of inputs"}

    out = {
        "metric": "multi-head SSM (state-space-duality form) fwd Gtok·ch/s and achieved HBM GB/s",
        "value": round(tok_ch / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"SSD layer: batch {b}, L {L}, {H} heads x head dim {P} (d_inner {H * P}), "
                               f"d_state {N}, bf16 io, D skip, no gate, final state, launches replayed from one "
                               "HIP graph", "batch": b, "seqlen": L, "nheads": H, "headdim": P, "d_state": N},
        "kernel_ms": round(launch_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": read_traffic(alg_bytes, PROFILE_TRAFFIC_SSD, KERNEL_SOURCES_SSD)},
        "mfma": {"achieved_tflops": round(tflops, 1), "peak_tflops": 2500.0, "frac": round(tflops / 2500.0, 4)},
        "cpu_baseline": cpu,
        "parity_sampled": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clock settles only after ~100 ms of sustained load, so the
    # defaults warm up for a few hundred steps before timing
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=2, help="workload index (forward configs 0-3)")
    ap.add_argument("--npw", type=int, default=0, help="states per wave (0 = library default)")
    ap.add_argument("--nchunks", type=int, default=0, help="time chunks (0 = library default)")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass of the forward config instead")
    ap.add_argument("--conv", action="store_true", help="time the causal conv1d + SiLU on the forward config's input")
    ap.add_argument("--conv-fused", action="store_true",
                    help="time the causal conv1d + SiLU fused into the forward scan (and the two separate launches)")
    ap.add_argument("--ssd", action="store_true",
                    help="time the multi-head SSM with a scalar decay per head (state-space-duality form)")
    ap.add_argument("--varlen", action="store_true",
                    help="time a variable-length batch with the forward config's channels and total tokens")
    ap.add_argument("--varlen-lens", default="",
                    help="varlen: comma-separated sequence lengths instead of the seeded 64-2048 mix")
    ap.add_argument("--dstate", type=int, default=0,
                    help="override the workload's d_state (up to 64; the headline workload uses 16)")
    ap.add_argument("--discretization", choices=["zoh", "euler"], default="zoh",
                    help="input term of the forward/decode workloads (zoh: the default, Euler: Delta B u)")
    ap.add_argument("--no-graph", action="store_true", help="conv: time eager launches (per-launch events) instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the scan shards over "
              "(batch, channel) with no communication, so the whole-job rate at N GPUs is N times the one-GPU "
              "rate of the per-GPU share -- run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import selective_state_space_55_amd as mscan
    from workloads import CONFIGS, forward_inputs, max_rel_err

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 3}))
        return 0

    if args.ssd:
        return bench_ssd(args)
    c = CONFIGS[args.config]
    if args.dstate:
        import dataclasses

        c = dataclasses.replace(c, dstate=args.dstate, name=f"{c.name} (d_state {args.dstate})")
    if c.kind == "step":
        return bench_step(args, c)
    if args.bwd:
        return bench_bwd(args, c)
    if args.conv:
        return bench_conv(args, c)
    if args.conv_fused:
        return bench_conv_fused(args, c)
    if args.varlen:
        return bench_varlen(args, c)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = forward_inputs(c)
    gen_s = time.time() - t0
    a = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    b, d, n, L = c.batch, c.dim, c.dstate, c.seqlen
    io = mscan.BF16 if c.io == "bf16" else mscan.F32
    ws_bytes = mscan.fwd_workspace_size(b, d, n, L, io, args.nchunks, args.npw)
    ws = torch.empty(max(ws_bytes, 1) + 256, dtype=torch.uint8, device=dev)
    y = torch.empty((b, d, L), dtype=a["u"].dtype, device=dev)
    fs = torch.empty((b, d, n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mscan.scan_fwd(a["u"], a["delta"], a["A_log"], a["B"], a["C"], D=a["D"], z=a["z"],
                       delta_bias=a["delta_bias"], out=y, final_state=fs, return_final_state=True,
                       workspace=ws, nchunks=args.nchunks, states_per_wave=args.npw, stream=stream,
                       discretization=args.discretization)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    launch_ms_avg = sum(launch_ms) / len(launch_ms)
    ms_per_step = wall * 1e3 / args.steps

    tc = b * d * L
    value = tc / (ms_per_step * 1e-3) / 1e9
    alg_bytes = c.algorithmic_bytes()
    hbm_gbps = alg_bytes / (launch_ms_avg * 1e-3) / 1e9
    per_tcn = SLOTS_PER_TCN if args.discretization == "zoh" else SLOTS_PER_TCN_EULER
    slots = tc * n * per_tcn + tc * (SLOTS_PER_TC_GATED if c.gated else SLOTS_PER_TC_UNGATED)
    achieved = slots / (launch_ms_avg * 1e-3) / 1e12
    peak = VALU_SLOTS_PEAK / 1e12
    # the committed counters were taken on the ZOH kernel at the workload's own d_state and the
    # default plan, per workload
    prof = PROFILE_TRAFFIC_FWD.get(args.config)
    default_plan = args.discretization == "zoh" and not args.dstate and not args.nchunks and not args.npw
    traffic = read_traffic(alg_bytes, prof) if (prof and default_plan) else None
    flushed = None
    if alg_bytes < CACHE_BYTES:
        # the workload fits the 256 MB Infinity Cache: also time launches that follow a 1 GiB
        # scratch write, so every input comes from HBM
        fl_ms = flushed_launch_ms(lambda r: step(), stream, max(11, min(args.steps, 50)))
        fl_gbps = alg_bytes / (fl_ms * 1e-3) / 1e9
        flushed = {"kernel_ms": round(fl_ms, 4), "value": round(tc / (fl_ms * 1e-3) / 1e9, 3),
                   "GBps": round(fl_gbps, 1), "frac_of_8TBps": round(fl_gbps / HBM_PEAK_GBPS, 4),
                   "note": "median launch after a 1 GiB scratch write (cold Infinity Cache); the figures "
                           "above are warm, back-to-back launches"}

    parity = None
    if not args.no_parity:
        import oracle

        rows = [0, d // 3, d - 1] if b == 1 else [0, d // 2 + 7, (b - 1) * d + d - 1]
        yg = y.view(b * d, L)[rows].cpu()
        fg = fs.view(b * d, n)[rows].cpu()
        errs = []
        for i, r in enumerate(rows):
            bb, dd = divmod(r, d)
            sub = dict(u=inp["u"][bb:bb + 1, dd:dd + 1], delta=inp["delta"][bb:bb + 1, dd:dd + 1],
                       A_log=inp["A_log"][dd:dd + 1], B=inp["B"][bb:bb + 1], C=inp["C"][bb:bb + 1],
                       D=None if inp["D"] is None else inp["D"][dd:dd + 1],
                       z=None if inp["z"] is None else inp["z"][bb:bb + 1, dd:dd + 1],
                       delta_bias=None if inp["delta_bias"] is None else inp["delta_bias"][dd:dd + 1])
            yr, fr = oracle.scan_fwd(**sub, discretization=args.discretization)
            errs.append((yr[0, 0], fr[0, 0]))
        parity = {
            "rows": rows,
            "y_max_rel": max_rel_err(yg, np.stack([e[0] for e in errs])),
            "final_state_max_rel": max_rel_err(fg, np.stack([e[1] for e in errs])),
            "tol": c.tol,
        }

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = host_cores()
        # bounded sample of the same workload: whole batch rows and channels, full length,
        # at most ~4e9 (token, channel, state) updates (a few seconds on 16 host cores)
        budget = 4e9
        nch = int(min(d, max(1, budget // (L * n))))
        nrow = int(min(b, max(1, budget // (nch * L * n))))
        per_ch = ("u", "delta", "z")
        sub = {}
        for k, v in inp.items():
            if v is None:
                sub[k] = None
            elif k in per_ch:
                sub[k] = v[:nrow, :nch]
            elif k in ("B", "C"):
                sub[k] = v[:nrow]
            elif k in ("A_log", "D", "delta_bias"):
                sub[k] = v[:nch]
            else:
                sub[k] = v
        c0 = time.perf_counter()
        oracle.scan_fwd(sub["u"], sub["delta"], sub["A_log"], sub["B"], sub["C"], D=sub["D"], z=sub["z"],
                        delta_bias=sub["delta_bias"], nthreads=cores, discretization=args.discretization)
        cs = time.perf_counter() - c0
        whole = "the whole workload" if (nrow == b and nch == d) else "a sample of the workload"
        cpu = {"value": round(nrow * nch * L / cs / 1e9, 6), "unit": "Gtok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"{whole}: {nrow} batch rows x {nch} channels x {L} tokens x {n} states, fp64, "
                         f"{cs:.2f} s wall incl. fp64 widening of inputs"}

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{c.name} selective-scan forward" + ("" if args.discretization == "zoh" else " (Euler)")
                        + f": batch {b}, d_inner {d}, d_state {n}, L {L}, "
                        f"{c.io} io, fp32 state, {'gated' if c.gated else 'ungated'}, final state",
            "batch": b, "d_inner": d, "d_state": n, "seqlen": L, "io": c.io, "gated": c.gated,
            "parallelism": "single GPU",
        },
        "kernel_ms": round(launch_ms_avg, 4),
        "hbm": {"algorithmic_bytes": alg_bytes, "GBps": round(hbm_gbps, 1),
                "frac_of_8TBps": round(hbm_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(peak, 3),
            "unit": "T fp32 lane-op slots/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "flushed": flushed,
        "cpu_baseline": cpu,
        "parity_sampled": parity,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
