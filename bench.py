#!/usr/bin/env python3
"""Benchmark of the per-chunk WY/UT preparation (kkt_solve + W/U) on one MI355X.

One step = one wy_prepare launch over the whole workload: every (chunk, value head) unit of
B=1, T=8192, Hq=Hv=16, d=128, C=64, bf16 k/v (fp32 beta, T out fp32, W/U out bf16).  Inputs
are seeded synthetic data, resident in HBM before the timed region.  Several copies of the
input/output buffers are rotated so that consecutive steps do not hit the 256 MB Infinity
Cache with the previous step's data.

Prints one JSON line.  value = units (chunk x value head) per second, from the GPU time of the
timed steps (one HIP event pair around them, on the launch stream); the roofline's achieved
bandwidth comes from the same figure.  The same run also times the other C = 64 workloads and
the chunk-size study (extra key "workloads"), each with its own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunks/s (tokens/s) for kkt_solve+W/U at C=64; achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 768 << 20  # rotated footprint: three times the Infinity Cache
CSRC = os.path.join(ROOT, "chunkwise_gated_deltanet_amd", "csrc")
# Kernel sources behind each entry point; a committed counter summary is used only while the
# hash of these files matches the one it was taken on.
KERNEL_SOURCES = {
    "wy": ("wyprep_device.h", "wyprep_kernels.hip"),
    "fwd": ("chunk_fwd.hip",),
    "bwd": ("wyprep_device.h", "wy_backward.hip"),
}
ENTRY_NAMES = {"wy": "wy_prepare", "wu": "wu_prepare", "kkt": "kkt_solve", "fwd": "chunk_fwd",
               "gdn": "gdn_forward", "bwd": "wy_backward", "solve": "solve_rhs"}


def algorithmic_bytes(tokens, hq, hv, dk, dv, C, esz, entry="wy", gated=False):
    """K read once per key head, beta (and g when gated) read once; wy: V read, T (fp32), W and
    U written once; wu: the same without T; kkt: T only; solve: one right-hand side R read and
    X written (R and X in the value-head layout, like V and U)."""
    gb = 4 if gated else 0
    if entry == "kkt":
        return tokens * (hq * dk * esz + hv * (4 + gb + 4 * C))
    if entry == "solve":
        return tokens * (hq * dk * esz + hv * (dv * esz + 4 + gb + dv * esz))
    t_bytes = 4 * C if entry == "wy" else 0
    per_token = hq * dk * esz + hv * (dv * esz + 4 + gb + t_bytes + dk * esz + dv * esz)
    return tokens * per_token


def fwd_bytes(tokens, num_states, hq, hv, dk, dv, esz, gated=False):
    """chunk_fwd: q and k read once per key head; W, U (and g) read, o written once per value
    head; the final state (fp32, dk x dv per sequence and value head) written once."""
    gb = 4 if gated else 0
    return tokens * (2 * hq * dk * esz + hv * (dk * esz + dv * esz + gb + dv * esz)) + \
        num_states * hv * dk * dv * 4


def bwd_bytes(tokens, hq, hv, dk, dv, esz, gated=False):
    """wy_backward without dT: k read and dk written once per key head; v, beta, dW, dU (and g)
    read, dv and dbeta (and dg) written once per value head."""
    gb = 8 if gated else 0
    return tokens * (2 * hq * dk * esz + hv * (3 * dv * esz + dk * esz + 8 + gb))


def kernel_source_sha(entry="wy"):
    """SHA-256 over the kernel sources of an entry point (wu, kkt, gdn: those of wy), in order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(entry, KERNEL_SOURCES["wy"]):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_name(entry, w, batch, seqlen, num_seqs, seg_chunks=None):
    """Name of the profiles/ summaries for one entry point and workload, e.g.
    wy_prepare_bf16_c64_b1t8192h16, wy_prepare_bf16_c64_packed8_hq16hv64, with log gates
    wy_prepare_gated_bf16_c64_b1t8192h16, or for the split forward (segments of 16 chunks)
    chunk_fwd_cp16_bf16_c64_b1t8192h16."""
    if num_seqs:
        shape = f"packed{num_seqs}_hq{w.num_qk_heads}hv{w.num_v_heads}"
    elif w.num_qk_heads == w.num_v_heads:
        shape = f"b{batch}t{seqlen}h{w.num_v_heads}"
    else:
        shape = f"b{batch}t{seqlen}hq{w.num_qk_heads}hv{w.num_v_heads}"
    gated = "_gated" if w.gate_mu is not None else ""
    split = f"_cp{seg_chunks}" if seg_chunks is not None and entry in ("fwd", "gdn") else ""
    return f"{ENTRY_NAMES[entry]}{split}{gated}_{w.dtype}_c{w.chunk_size}_{shape}"


def counter_traffic(name, entry="wy"):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this entry point
    and workload, if there is one and it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", name + "_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m_b or not m_h or m_h.group(1) != kernel_source_sha(entry):
        return None
    return float(m_b.group(1))


def host_cores():
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_threads():
    """Threads for the CPU baseline: every usable host core, at most 16 (one GPU's share of a
    GPU machine's cores; the rest belong to the other GPUs of the machine)."""
    return max(1, min(16, host_cores()))


def cpu_baseline(inp, units_per_pass, tokens_per_pass, seconds=10.0, entry="wy"):
    """The fp64 oracle, as it stands, on the same workload: whole passes until ~`seconds` on
    every usable host core, then until ~`seconds`/3 on one core.  entry "solve" times the
    oracle's right-hand-side solve with v as the right-hand side; every other entry the whole
    preparation (T, W, U)."""
    import oracle
    lib = oracle.load()

    def timed(threads, budget):
        passes, t0 = 0, time.perf_counter()
        while True:
            if entry == "solve":
                oracle.solve_rhs(inp["k"], inp["v"], inp["beta"], inp["chunk_size"],
                                 cu_seqlens=inp["cu_seqlens"], g=inp["g"], nthreads=threads,
                                 lib=lib)
            else:
                oracle.wy_prepare(inp["k"], inp["beta"], inp["chunk_size"], v=inp["v"],
                                  cu_seqlens=inp["cu_seqlens"], nthreads=threads, lib=lib,
                                  g=inp["g"])
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return passes, el

    threads = cpu_threads()
    passes, el = timed(threads, seconds)
    passes1, el1 = timed(1, seconds / 3)
    return {"value": units_per_pass * passes / el, "unit": "chunks/s", "cores": threads,
            "host_cores": host_cores(), "kind": "oracle",
            "sample": f"whole workload ({units_per_pass} units, {tokens_per_pass} tokens) x "
                      f"{passes} passes, {el:.1f} s wall, fp64; one core: {passes1} passes, "
                      f"{el1:.1f} s",
            "tokens_per_s": tokens_per_pass * passes / el,
            "value_one_core": units_per_pass * passes1 / el1}


def cpu_baseline_bwd(inp, units_per_pass, tokens_per_pass, workload, seconds=10.0):
    """The fp64 backward oracle, as it stands, on the whole workload (the same seeded dW, dU):
    whole passes until ~`seconds` on every usable host core."""
    import oracle
    from chunkwise_gated_deltanet_amd import synth
    lib = oracle.load()
    threads = cpu_threads()
    B, T, Hv = inp["beta"].shape
    grng = np.random.default_rng(1000 + workload)
    dW = synth.f32_to_bf16_bits(grng.standard_normal((B, T, Hv, 128), dtype=np.float32))
    dU = synth.f32_to_bf16_bits(grng.standard_normal((B, T, Hv, 128), dtype=np.float32))
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.wy_backward(inp["k"], inp["v"], inp["beta"], inp["chunk_size"], dW, dU,
                           g=inp["g"], cu_seqlens=inp["cu_seqlens"], nthreads=threads, lib=lib)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": units_per_pass * passes / el, "unit": "chunks/s", "cores": threads,
            "host_cores": host_cores(), "kind": "oracle",
            "sample": f"whole workload ({units_per_pass} units, {tokens_per_pass} tokens) x "
                      f"{passes} passes, {el:.1f} s wall, fp64 backward",
            "tokens_per_s": tokens_per_pass * passes / el}


def cpu_baseline_fwd(inp, seconds=10.0):
    """The token-by-token fp64 recurrence oracle, as it stands, on a bounded sample of the
    workload: the first (sequence, value head) pairs, one per usable host core, repeated until
    ~`seconds`; reported per chunk x value head of those pairs."""
    import oracle
    lib = oracle.load()
    threads = cpu_threads()
    B, T, C = inp["batch"], inp["seqlen"], inp["chunk_size"]
    Hv = inp["beta"].shape[2]
    cu = inp["cu_seqlens"]
    N = B if cu is None else len(cu) - 1
    lens = np.full(N, T) if cu is None else np.diff(cu.astype(np.int64))
    pairs = [(p // Hv, p % Hv) for p in range(min(threads, N * Hv))]
    units = int(sum((lens[s] + C - 1) // C for s, _ in pairs))
    toks = int(sum(lens[s] for s, _ in pairs))
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"],
                           cu_seqlens=cu, pairs=pairs, nthreads=threads, lib=lib)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": units * passes / el, "unit": "chunks/s", "cores": threads,
            "host_cores": host_cores(), "kind": "oracle",
            "sample": f"{len(pairs)} (sequence, value head) pairs ({units} chunk x head units, "
                      f"{toks} tokens each pass) x {passes} passes, {el:.1f} s wall, fp64 "
                      "token-by-token recurrence",
            "tokens_per_s": toks * passes / el}


# Extra workloads timed after the headline (each with its own roofline): the other C = 64
# configurations, the chunk-size study on B=4 T=4096 H=32, 1024 short packed sequences (the
# packed-sequence work map under load), and on the headline's shape the backward at C = 64, 32
# and 128 and the chunk recurrence in its sequence-parallel form.
DEFAULT_EXTRAS = "3:32,3:64,3:128,5:64,6:64,bwd/2:64,bwd/2:32,bwd/2:128,fwd/2:64/auto"


def parse_extras(text, entry="wy"):
    """'[entry/]workload:C[/segments]' items, comma-separated, -> (entry, workload, C, segments)
    tuples; the entry defaults to `entry`, segments (fwd / gdn: an int or 'auto') to None.
    'none' or '' -> []."""
    if not text or text == "none":
        return []
    out = []
    for item in text.split(","):
        parts = item.split("/")
        e = entry
        if not parts[0][:1].isdigit():
            e = parts.pop(0)
            if e not in ENTRY_NAMES:
                raise ValueError(f"unknown entry point in extras item {item!r}")
        idx, c = parts[0].split(":")
        seg = parts[1] if len(parts) > 1 else None
        out.append((e, int(idx), int(c), seg))
    return out


def measure(args, entry, w, inp, dev, lib, ramp=True):
    """Times `args.steps` steps of one entry point on one workload; returns the result fields
    (and the timing details) as a dict."""
    import ctypes
    import torch
    import chunkwise_gated_deltanet_amd as cg
    from chunkwise_gated_deltanet_amd import synth

    fwd_entry = entry in ("fwd", "gdn")
    bwd_entry = entry == "bwd"
    gated = inp["g"] is not None
    B, T = inp["batch"], inp["seqlen"]
    Hq, Hv, C = w.num_qk_heads, w.num_v_heads, w.chunk_size
    dk = dv = 128
    esz = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if inp["cu_seqlens"] is not None:
        lens = np.diff(inp["cu_seqlens"].astype(np.int64))
        nchunks = int(np.sum((lens + C - 1) // C))
    else:
        nchunks = B * ((T + C - 1) // C)
    units = nchunks * Hv
    tokens = B * T
    nstates = B if inp["cu_seqlens"] is None else len(inp["cu_seqlens"]) - 1
    if entry == "bwd":
        alg = bwd_bytes(tokens, Hq, Hv, dk, dv, esz, gated)
    elif entry == "fwd":
        alg = fwd_bytes(tokens, nstates, Hq, Hv, dk, dv, esz, gated)
    elif entry == "gdn":
        alg = algorithmic_bytes(tokens, Hq, Hv, dk, dv, C, esz, "wu", gated) + \
            fwd_bytes(tokens, nstates, Hq, Hv, dk, dv, esz, gated)
    else:
        alg = algorithmic_bytes(tokens, Hq, Hv, dk, dv, C, esz, entry, gated)
    nsets = max(1, math.ceil(ROTATE_BYTES / alg))  # every byte of a step is touched once

    def dev_tensor(a, dt):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        return (t.view(torch.bfloat16) if dt == torch.bfloat16 else t).to(dev)

    k0 = dev_tensor(inp["k"], tdt)
    v0 = dev_tensor(inp["v"], tdt)
    b0 = torch.from_numpy(inp["beta"]).to(dev)
    g0 = torch.from_numpy(inp["g"]).to(dev) if gated else None
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(dev)
    q0 = dev_tensor(inp["q"], tdt) if fwd_entry else None
    if bwd_entry:  # upstream gradients dW, dU: seeded N(0, 1), bf16
        grng = np.random.default_rng(1000 + args.workload)
        dW0 = dev_tensor(synth.f32_to_bf16_bits(grng.standard_normal((B, T, Hv, dk), dtype=np.float32)), tdt)
        dU0 = dev_tensor(synth.f32_to_bf16_bits(grng.standard_normal((B, T, Hv, dv), dtype=np.float32)), tdt)
    sets = []
    for i in range(nsets):
        first = i == 0  # set 0 uses the uploaded tensors themselves
        sets.append(dict(k=k0 if first else k0.clone(), v=v0 if first else v0.clone(),
                         beta=b0 if first else b0.clone(),
                         g=(g0 if first else g0.clone()) if gated else None,
                         T=torch.empty(B, T, Hv, C, dtype=torch.float32, device=dev)
                         if entry in ("wy", "kkt") else None,
                         W=torch.empty(B, T, Hv, dk, dtype=tdt, device=dev)
                         if entry not in ("kkt", "solve") else None,
                         U=torch.empty(B, T, Hv, dv, dtype=tdt, device=dev)
                         if entry != "kkt" else None,  # solve: X
                         q=(q0 if first else q0.clone()) if fwd_entry else None,
                         o=torch.empty(B, T, Hv, dv, dtype=tdt, device=dev) if fwd_entry else None,
                         hT=torch.empty(nstates, Hv, dk, dv, dtype=torch.float32, device=dev)
                         if fwd_entry else None,
                         dW=(dW0 if first else dW0.clone()) if bwd_entry else None,
                         dU=(dU0 if first else dU0.clone()) if bwd_entry else None,
                         dk=torch.empty_like(k0) if bwd_entry else None,
                         dv=torch.empty_like(v0) if bwd_entry else None,
                         db=torch.empty_like(b0) if bwd_entry else None,
                         dg=torch.empty_like(b0) if bwd_entry and gated else None))
    prob = cg.Problem(B, T, Hq, Hv, dk, dv, C, 0 if cu is None else cu.numel() - 1,
                      0 if w.dtype == "bf16" else 1)
    pprob = ctypes.byref(prob)
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    calls = [tuple(ctypes.c_void_p(None if t is None else t.data_ptr()) for t in
                   (s["k"], s["v"], s["g"], s["beta"], s["T"], s["W"], s["U"], s["q"], s["o"],
                    s["hT"])) for s in sets]
    bcalls = [tuple(ctypes.c_void_p(None if t is None else t.data_ptr()) for t in
                    (s["dW"], s["dU"], s["dk"], s["dv"], s["db"], s["dg"])) for s in sets]
    cu_ptr = ctypes.c_void_p(None if cu is None else cu.data_ptr())
    scale = ctypes.c_float(dk ** -0.5)
    seg_chunks = None
    if fwd_entry and args.segment_chunks is not None:
        seg_chunks = (cg.auto_segment_chunks(B, T, Hv, C, None if cu is None else cu.numel() - 1)
                      if args.segment_chunks == "auto" else int(args.segment_chunks))
    if seg_chunks is not None:
        ws_bytes = lib.wyp_chunk_fwd_cp_workspace_bytes(pprob, cu_ptr, seg_chunks)
        ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev)
        ws_ptr, ws_n = ctypes.c_void_p(ws.data_ptr()), ctypes.c_int64(ws_bytes)

    def step(i, sp):
        kp, vp, gp, bp, tp, wp, up, qp, op, hp = calls[i % nsets]
        if entry == "wy":
            st = lib.wyp_wy_prepare(pprob, kp, vp, gp, bp, cu_ptr, tp, wp, up, sp)
        elif entry == "wu":
            st = lib.wyp_wu_prepare(pprob, kp, vp, gp, bp, cu_ptr, wp, up, sp)
        elif entry == "kkt":
            st = lib.wyp_kkt_solve(pprob, kp, gp, bp, cu_ptr, tp, sp)
        elif entry == "solve":  # the right-hand side is v, X goes to the U buffer
            st = lib.wyp_solve_rhs(pprob, kp, vp, gp, bp, cu_ptr, up, sp)
        elif entry == "bwd":
            dwp, dup, dkp, dvp, dbp, dgp = bcalls[i % nsets]
            st = lib.wyp_wy_backward(pprob, kp, vp, gp, bp, cu_ptr, None, dwp, dup, dkp, dvp, dbp,
                                     dgp, sp)
        else:
            st = 0
            if entry == "gdn":
                st = lib.wyp_wu_prepare(pprob, kp, vp, gp, bp, cu_ptr, wp, up, sp)
            if st == 0 and seg_chunks is not None:
                st = lib.wyp_chunk_fwd_cp(pprob, qp, kp, wp, up, gp, None, scale, cu_ptr,
                                          seg_chunks, ws_ptr, ws_n, op, hp, sp)
            elif st == 0:
                st = lib.wyp_chunk_fwd(pprob, qp, kp, wp, up, gp, None, scale, cu_ptr, op, hp, sp)
        if st != 0:
            raise RuntimeError(lib.wyp_last_error().decode())

    if entry == "fwd":  # W and U of every buffer set, prepared once, untimed
        for i in range(nsets):
            kp, vp, gp, bp, tp, wp, up, qp, op, hp = calls[i]
            if lib.wyp_wu_prepare(pprob, kp, vp, gp, bp, cu_ptr, wp, up, sptr) != 0:
                raise RuntimeError(lib.wyp_last_error().decode())
        torch.cuda.synchronize(dev)

    # Clock ramp: the GPU needs ~20 ms of sustained work to reach steady clocks (measured on
    # this kernel: 43 us per launch in the first 4 ms, 30 us from 20 ms on).  The step runs
    # untimed for at least --ramp-ms before the counted warm-up steps; the count is reported.
    ramp_launches = 0
    if ramp:
        t_end = time.perf_counter() + args.ramp_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(50):
                step(ramp_launches, sptr)
                ramp_launches += 1
            torch.cuda.synchronize(dev)
    for i in range(args.warmup):
        step(i, sptr)
    torch.cuda.synchronize(dev)

    # The K launches of the timed region are captured once into a HIP graph (unless --eager):
    # one host call then submits all of them, so the host's per-launch cost (ctypes, argument
    # checks, hipLaunchKernel) cannot leave the GPU idle between these ~30 us kernels.
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream(dev)):
            csp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            for i in range(args.steps):
                step(i, csp)
        graph.replay()  # untimed: the first replay also uploads the graph
        torch.cuda.synchronize(dev)

    # The outputs the last timed launch writes are filled with NaN first, so the check after
    # the timed region fails if the timed launches did not write them.
    last = (args.steps - 1) % nsets
    outs = {"wy": ("T", "W", "U"), "wu": ("W", "U"), "kkt": ("T",), "solve": ("U",),
            "fwd": ("o", "hT"),
            "gdn": ("W", "U", "o", "hT"),
            "bwd": ("dk", "dv", "db") + (("dg",) if gated else ())}[entry]
    for n in outs:
        sets[last][n].fill_(float("nan"))

    # Timed region: exactly `steps` launches, one event pair around them on the launch stream
    # (an event pair per launch would add its own few microseconds to each).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i, sptr)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_s = e0.elapsed_time(e1) * 1e-3 / args.steps  # GPU seconds per step, gaps included

    # The timed launches did the work: the outputs of the last buffer set hold no NaN and equal
    # a fresh eager launch bit for bit.
    got = {n: sets[last][n].clone() for n in outs}
    written = all(not torch.isnan(got[n]).any() for n in outs)
    step(last, sptr)
    torch.cuda.synchronize(dev)
    replay_ok = written and all(torch.equal(got[n], sets[last][n]) for n in outs)

    # Diagnostic only (after the timed region): spread of single eager launches, each between
    # its own pair of events, so every figure carries one event pair's overhead.
    nd = min(args.steps, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nd)]
    for i in range(nd):
        ev[i][0].record(stream)
        step(i, sptr)
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3

    achieved = alg / step_s / 1e9
    pname = profile_name(entry, w, B, T, 0 if cu is None else cu.numel() - 1, seg_chunks)
    traffic = counter_traffic(pname, entry) if entry != "gdn" else None
    res = {
        "units": units, "tokens": tokens, "alg": alg, "nsets": nsets, "seg_chunks": seg_chunks,
        "ramp_launches": ramp_launches, "launch": "eager" if graph is None else
        "hip graph of the timed launches", "replay_ok": replay_ok, "step_s": step_s,
        "wall_s": wall,
        "kernel_us": {"mean": step_s * 1e6,
                      "single_launch_p10": float(np.percentile(durs, 10)) * 1e6,
                      "single_launch_p50": float(np.median(durs)) * 1e6,
                      "single_launch_p90": float(np.percentile(durs, 90)) * 1e6},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes": alg},
    }
    del sets, graph
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--ramp-ms", type=float, default=100.0,
                    help="untimed launches for at least this long before the warm-up steps, so "
                         "the GPU clocks are steady (0 = none)")
    ap.add_argument("--workload", type=int, default=2,
                    help="seeded workload index (2 = the headline C=64 workload)")
    ap.add_argument("--chunk-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--entry", choices=("wy", "wu", "kkt", "solve", "fwd", "gdn", "bwd"),
                    default="wy",
                    help="wy: wyp_wy_prepare (T, W, U; the headline); wu: wyp_wu_prepare "
                         "(W, U, no T in HBM); kkt: wyp_kkt_solve (T only); solve: "
                         "wyp_solve_rhs with v as the one right-hand side (X = U, T never "
                         "formed); fwd: wyp_chunk_fwd "
                         "(state recurrence and output from prepared W, U; C = 32, 64, 128); gdn: the "
                         "whole forward, wyp_wu_prepare then wyp_chunk_fwd; bwd: "
                         "wyp_wy_backward (dk, dv, dbeta, dg from dW, dU; no dT; C = 64)")
    ap.add_argument("--gate-mu", type=float, default=None,
                    help="add per-token log gates g = log sigmoid(mu + N(0,1)) (the gated "
                         "coefficient diag(beta)(Gamma o K K^T)); 4 is the seeded gated recipe")
    ap.add_argument("--segment-chunks", default=None,
                    help="fwd / gdn entries: split each sequence into segments of this many "
                         "chunks run in parallel (wyp_chunk_fwd_cp); 'auto' picks it from the "
                         "shape")
    ap.add_argument("--extras", default=None,
                    help="extra workloads timed after the main one, comma-separated "
                         "[entry/]workload:C[/segments] items (the entry defaults to --entry; "
                         "segments for fwd / gdn: chunks per segment or 'auto'); default for "
                         f"the headline: {DEFAULT_EXTRAS}; 'none' for none")
    ap.add_argument("--eager", action="store_true",
                    help="launch each timed step from Python instead of replaying a graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE against known bytes)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the preparation step has no cross-GPU exchange, "
              "so N GPUs would each run the same kernel on their own share of the heads or "
              "chunks (use --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import chunkwise_gated_deltanet_amd as cg
    from chunkwise_gated_deltanet_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    lib = cg.load_library()

    fwd_entry = args.entry in ("fwd", "gdn")
    w = synth.workload(args.workload, chunk_size=args.chunk_size, gate_mu=args.gate_mu,
                       with_q=fwd_entry)
    if args.gate_mu is not None:
        w.name += f" gated (g = log sigmoid({args.gate_mu:g} + N(0,1)))"
    inp = synth.generate(w)
    gated = inp["g"] is not None
    B, T = inp["batch"], inp["seqlen"]
    C = w.chunk_size
    r = measure(args, args.entry, w, inp, dev, lib, ramp=True)
    units, tokens = r["units"], r["tokens"]
    out = {
        "metric": METRIC if args.entry == "wy" else f"chunks/s (tokens/s) for {ENTRY_NAMES[args.entry]} at C={C}; achieved HBM GB/s vs peak",
        "value": units / r["step_s"],
        "unit": "chunks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "entry": ENTRY_NAMES[args.entry], "gated": gated,
                   "segment_chunks": r["seg_chunks"] if fwd_entry else None,
                   "batch": B, "seqlen": T, "num_qk_heads": w.num_qk_heads,
                   "num_v_heads": w.num_v_heads, "head_dim": 128, "chunk_size": C,
                   "units_per_step": units, "tokens_per_step": tokens,
                   "rotated_buffer_sets": r["nsets"], "launch": r["launch"],
                   "clock_ramp_launches": r["ramp_launches"],
                   "replay_matches_eager": r["replay_ok"],
                   "timing": "ms_per_step, value and roofline.achieved come from one HIP event "
                             "pair around the timed launches on the launch stream"},
        "tokens_per_s": tokens / r["step_s"],
        "host_wall_ms_per_step": r["wall_s"] * 1e3 / args.steps,
        "kernel_us": r["kernel_us"],
        "roofline": r["roofline"],
        "cpu_baseline": None,
    }
    if args.entry == "gdn":
        out["roofline"]["note"] = ("two kernels per step (wu_prepare, chunk_fwd): achieved is "
                                   "their summed algorithmic bytes over the step time")
    extras = parse_extras(args.extras if args.extras is not None else
                          (DEFAULT_EXTRAS if args.entry == "wy" and args.workload == 2 and
                           args.chunk_size in (None, 64) and not gated else "none"), args.entry)
    if extras:
        out["workloads"] = []
        cache = {}
        for e, idx, c, seg in extras:
            e_fwd = e in ("fwd", "gdn")
            we = synth.workload(idx, chunk_size=c, gate_mu=args.gate_mu, with_q=e_fwd)
            # the chunk size changes only a packed workload's lengths
            key = (idx, c if we.seq_range is not None else None, e_fwd)
            if key not in cache:
                cache.clear()
                cache[key] = synth.generate(we)
            ie = dict(cache[key], chunk_size=c)
            args_e = argparse.Namespace(**vars(args))
            args_e.workload, args_e.segment_chunks = idx, (seg if e_fwd else None)
            # each gets its own clock ramp: the GPU idles while the host draws its inputs
            re_ = measure(args_e, e, we, ie, dev, lib, ramp=True)
            out["workloads"].append({
                "workload": we.name, "entry": ENTRY_NAMES[e], "chunk_size": c,
                "segment_chunks": re_["seg_chunks"] if e_fwd else None,
                "units_per_step": re_["units"],
                "tokens_per_step": re_["tokens"], "ms_per_step": re_["step_s"] * 1e3,
                "value": re_["units"] / re_["step_s"], "unit": "chunks/s",
                "tokens_per_s": re_["tokens"] / re_["step_s"],
                "replay_matches_eager": re_["replay_ok"], "rotated_buffer_sets": re_["nsets"],
                "clock_ramp_launches": re_["ramp_launches"],
                "kernel_us": re_["kernel_us"], "roofline": re_["roofline"]})
        cache.clear()
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
    if not args.no_cpu_baseline:
        if fwd_entry:
            out["cpu_baseline"] = cpu_baseline_fwd(inp, args.cpu_seconds)
        elif args.entry == "bwd":
            out["cpu_baseline"] = cpu_baseline_bwd(inp, units, tokens, args.workload,
                                                   args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(inp, units, tokens, args.cpu_seconds, args.entry)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
