#!/usr/bin/env python3
"""Benchmark of the MI355X selective-scan forward (one GPU).

One step = one ss_fwd call over one batch of synthetic input already resident in
HBM: the fused scan (B/C tiles through LDS, softplus step size, exp discretisation,
recurrence, readout, D skip, SiLU gate), i.e. every forward row of the hot path.
For the fwd+bwd workload (--workload c4) a step is ss_fwd followed by ss_bwd.
Default workload: S6 fwd + gate, bf16 x/z/dt_raw/B/C, fp32 A/D/dt_bias/state/y,
B=8 L=2048 D=5120 N=16.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value        B·L·D elements/s over the timed steps
  roofline     the scan kernel against its binding roof (the VALU issue rate: 256 CUs x
               4 SIMDs x 16 lanes x 2.4 GHz, packed fp32 unused), with its measured HBM
               traffic while the sources match the profiled ones, and the HBM view
               (minimum bytes / time vs 8 TB/s) beside it
  cpu_baseline the fp64 C oracle on a bounded sample of the same workload, host cores
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# ALU roof: 256 CUs x 4 SIMDs x 16 fp32 lanes x 2.4 GHz = 39.32e12 VALU lane-slots/s
# (packed fp32 is not used).  Measured on the part: a wave64 v_fma_f32 occupies its SIMD for
# one issue unit (full rate), a v_exp_f32 for two (half rate, 2 slots), and the two never
# overlap (active VALU units = FMAs + 2 x exps, VALU 100 % busy, in every mix).
ALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12


# HBM traffic of the dominant kernel per launch, from two rocprofv3 counter passes
# (FETCH_SIZE, WRITE_SIZE) that each also ran a 1 GiB device copy: the copy reads
# FETCH_SIZE = 512 MiB and WRITE_SIZE = 1 GiB, so reads = 2.0 x FETCH_SIZE and writes =
# 1.0 x WRITE_SIZE.  A figure is reported only while the kernel's sources hash to the
# value it was measured with; after any change it is null until measured again.
FWD_SOURCES = ["ss_fwdg.hip", "ss_device.h", "ss_plan.h", "ss_api.cpp", "ss_kernels.h"]
STEP_SOURCES = ["ss_step.hip", "ss_device.h", "ss_plan.h", "ss_api.cpp", "ss_kernels.h"]
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
MEASURED_TRAFFIC = {
    # (workload, disc): first-order (0) or exact zero-order hold (1)
    ("c2", 0): {"sources": FWD_SOURCES, "fetch_kib": 336256, "write_kib": 400152,
                "sources_sha256": "c40b06c7bcb4217afb7d5fafdf1bedf826f1e5e7ab38e00b8fc475d68368e828"},
    ("c2", 1): {"sources": FWD_SOURCES, "fetch_kib": 350292, "write_kib": 414831,
                "sources_sha256": "c40b06c7bcb4217afb7d5fafdf1bedf826f1e5e7ab38e00b8fc475d68368e828"},
    ("d1", 0): {"sources": STEP_SOURCES, "fetch_kib": 45069, "write_kib": 87040,
                "sources_sha256": "450fdbf9aa09ccccb4f2de494aa94e655b524ae1d714af9917a7ae57032b0ae4"},
}


def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "selective_state_space_34_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(w, disc=0):
    m = MEASURED_TRAFFIC.get((w.name, disc))
    if m is None or w.backward or m["sources_sha256"] != sources_sha256(m["sources"]):
        return None
    return FETCH_SCALE * m["fetch_kib"] * 1024 + WRITE_SCALE * m["write_kib"] * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def emit(out, value_key="value"):
    """Print the one JSON line: adds the library's build identity (the SHA-256 of the sources
    it was built from; load() has already refused any other) and, when the CPU oracle was
    timed, the GPU/CPU throughput ratio inside cpu_baseline (vs_baseline stays null: the pages
    publish no number for this metric)."""
    import selective_state_space_34_amd as ss
    out["build_id"] = ss.load().ss_build_id().decode()
    cpu = out.get("cpu_baseline")
    if cpu:
        cpu["gpu_over_cpu"] = out[value_key] / cpu["value"]
    print(json.dumps(out), flush=True)


def min_bytes(w, s_in, dt_shared=False):
    """Algorithmic HBM bytes of one forward: read x, dt_raw (, z), B, C and parameters,
    write y (the (B,L,D,N) state and Ā/B̄ are never materialised).  A shared Δraw is
    B·L values instead of B·L·D."""
    BLD = w.batch * w.seqlen * w.dim
    n_in = (3 if w.gate else 2) - (1 if dt_shared else 0)
    rd = n_in * BLD * s_in + 2 * w.batch * w.dstate * w.seqlen * s_in
    rd += w.batch * w.seqlen * s_in if dt_shared else 0
    rd += w.dim * w.dstate * 4 + 2 * w.dim * 4
    wr = BLD * 4 + (w.batch * w.dim * w.dstate * 4 if w.h_final else 0)
    return rd + wr


def bwd_min_bytes(w, s_in, dt_shared=False):
    """Algorithmic HBM bytes of one backward: read x, dt_raw, z (s_in), dy (4), B, C and the
    parameters; write dx, dt_raw-grad, dz (4 each), dB, dC (4·B·N·L each), dA, dD, ddt_bias.
    A shared Δraw and its gradient are B·L values each."""
    BLD = w.batch * w.seqlen * w.dim
    BL = w.batch * w.seqlen
    BNL = w.batch * w.dstate * w.seqlen
    n_in = 3 if w.gate else 2
    n_seq = n_in - (1 if dt_shared else 0)
    rd = n_seq * BLD * s_in + BLD * 4 + 2 * BNL * s_in + w.dim * w.dstate * 4 + 2 * w.dim * 4
    wr = n_seq * BLD * 4 + 2 * BNL * 4 + w.dim * w.dstate * 4 + 2 * w.dim * 4
    if dt_shared:
        rd += BL * s_in
        wr += BL * 4
    return rd + wr


def pow_a(w):
    """The workload's A is -(n+1) for every channel (unperturbed), so Ā_n = r^(n+1), r = e^{-δ}."""
    return not w.a_perturb


def alu_slots_per_elem(w, disc=0):
    """Algorithmic VALU lane-slots per (b,t,d) element (transcendental = 2 slots).
    Per state: exp (2) + δ·A, δx·B, state fma, readout fma (4)  -> 6 x N.
    With A = -(n+1) (first-order hold) each Ā is one product of the previous one and
    r = e^{-δ}: per state 4 (Ā product, δx·B, state fma, readout fma), per element r (3).
    The exact zero-order hold adds, at its cheapest, Ā - 1, x/A_n and one product per state
    (3; 1/A_n is a per-channel constant) -> 9 x N.
    Per element: softplus 5 VALU + 2 trans; δ·x 1; D·x fma 1; gate 4 VALU + 2 trans (if any);
    bf16 widening 1 per bf16 input tensor."""
    if disc:
        per_state = 9 * w.dstate
    elif pow_a(w):
        per_state = 4 * w.dstate + 3
    else:
        per_state = 6 * w.dstate
    elem = 5 + 2 * 2 + 1 + 1
    if w.gate:
        elem += 4 + 2 * 2
    if w.dtype == "bf16":
        elem += 3 if w.gate else 2
    return per_state + elem


def bwd_alu_slots_per_elem(w, disc=0):
    """Algorithmic VALU lane-slots per element of the backward (transcendental = 2 slots).
    Per state: recompute h (δ·A, exp 2, δx·B, FMA: 5); adjoint g += ds·C (1), dC term ds·h (1),
    dB term g·δx (1), Σ g·B (1), g·Ā·h_prev (2), dA FMA (1), Σ A·g·Ā·h_prev (1), g *= Ā (1);
    the channel sums of dB and dC (2) -> 17 x N.  The exact zero-order hold adds per state its
    gain in the recompute and again in the adjoint (3 + 3, as in the forward), ∂g/∂A from the
    gain (2), x·g (1), g·B apart from its sum (1), g·B·x (1) and its FMAs into dA and dδ (2)
    -> 30 x N.  Per element: softplus 9, sigmoid(u) 4, dx 2, dΔ 2, dD 1, with a gate
    sigmoid(z) 4 + ds 2 + dz 5; bf16 widening per bf16 input.  With A = -(n+1) (first-order
    hold) the recompute forms each Ā as one product of the previous one and r = e^{-δ}: 15 per
    state, plus r (3) per element."""
    elem = 9 + 4 + 2 + 2 + 1
    if w.gate:
        elem += 4 + 2 + 5
    if w.dtype == "bf16":
        elem += 3 if w.gate else 2
    if disc:
        return 30 * w.dstate + elem
    if pow_a(w):
        return 15 * w.dstate + 3 + elem
    return 17 * w.dstate + elem


def cpu_baseline(w, inp, budget_s=4.0, disc=0):
    """Time the fp64 C oracle (as it stands) on a growing sample of channels until
    one run takes about budget_s seconds of wall time on all host threads."""
    from oracle import cref
    threads = cref.threads(0)
    if w.backward:
        return cpu_baseline_fwd_bwd(w, inp, budget_s, disc, threads)
    C = w.batch * w.dim
    n = max(1, min(C, 64))
    rng = np.random.default_rng(0)
    args = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    def run(chans):
        # the decode step starts from the carried state and produces the next one
        cref.fwd(*args, z=inp.z if w.gate else None, h0=inp.h0 if w.decode else None,
                 chans=chans, want_h_final=w.decode, zoh=bool(disc))

    while True:
        chans = np.sort(rng.choice(C, n, replace=False))
        t0 = time.perf_counter()
        run(chans)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n == C:
            break
        n = min(C, int(n * max(2.0, budget_s / max(dt, 1e-3) / 2)))
    # a whole workload that runs in under a second is repeated until about a second
    reps = 1 if dt >= budget_s / 4 else int(np.ceil(budget_s / 4 / max(dt, 1e-4)))
    if reps > 1:
        t0 = time.perf_counter()
        for _ in range(reps):
            run(chans)
        dt = time.perf_counter() - t0
    elems = n * w.seqlen
    return {"value": reps * elems / dt, "unit": "elem/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {C} channels x full L={w.seqlen} (B*L*D elements {elems})"
                      f"{f' x {reps} runs' if reps > 1 else ''}, {dt:.2f} s wall on {threads} "
                      f"OpenMP threads"}


def cpu_baseline_fwd_bwd(w, inp, budget_s, disc, threads):
    """Forward + backward workloads: time the oracle's forward and then its backward (which
    recomputes the states itself, as the GPU backward does) on the first n channels of every
    batch row, n growing until one fwd+bwd takes about budget_s / 4 seconds."""
    from oracle import cref
    n = max(1, min(w.dim, 64))

    def run(n):
        sl = lambda a: np.ascontiguousarray(a[:, :n])
        x, dtr, dy = sl(inp.x), sl(inp.dt_raw), sl(inp.dy)
        z = sl(inp.z) if w.gate else None
        par = (inp.dt_bias[:n], inp.A[:n], inp.Bm, inp.Cm, inp.Dskip[:n])
        t0 = time.perf_counter()
        cref.fwd(x, dtr, *par, z=z, want_h_final=False, zoh=bool(disc))
        cref.bwd(x, dtr, *par, dy, z=z, zoh=bool(disc))
        return time.perf_counter() - t0

    while True:
        dt = run(n)
        if dt >= budget_s / 4 or n == w.dim:
            break
        n = min(w.dim, int(n * max(2.0, budget_s / max(dt, 1e-3) / 2)))
    # a whole workload that runs in under a second is repeated until about a second
    reps = 1 if dt >= budget_s / 4 else int(np.ceil(budget_s / 4 / max(dt, 1e-4)))
    if reps > 1:
        dt = sum(run(n) for _ in range(reps))
    elems = w.batch * n * w.seqlen
    return {"value": reps * elems / dt, "unit": "elem/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd + bwd on {w.batch} x {n} of {w.batch} x {w.dim} channels x full "
                      f"L={w.seqlen} (B*L*D elements {elems})"
                      f"{f' x {reps} runs' if reps > 1 else ''}, {dt:.2f} s of oracle time on "
                      f"{threads} OpenMP threads"}


def step_min_bytes(w, s_in, dt_shared=False):
    """Algorithmic HBM bytes of one decode step: read x, dt_raw (, z) [B, D] (a shared dt_raw:
    [B]), B, C [B, N] and the parameters, read and write the state [B, D, N], write y [B, D]."""
    BD = w.batch * w.dim
    n_in = (3 if w.gate else 2) - (1 if dt_shared else 0)
    return (n_in * BD * s_in + (w.batch * s_in if dt_shared else 0)
            + 2 * w.batch * w.dstate * s_in + w.dim * (w.dstate + 2) * 4
            + 2 * BD * w.dstate * 4 + BD * 4)


def run_decode(args, w, inp):
    """Decode workload: K timed ss_step calls, each carrying every (batch row, channel) one
    token further with the state updated in place.  Roofline: HBM (state in and out)."""
    import torch
    import selective_state_space_34_amd as ss
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    col = lambda a: torch.from_numpy(np.ascontiguousarray(a[..., 0])).to(dt).to(dev)
    t32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    x, Bm, Cm = col(inp.x), col(inp.Bm), col(inp.Cm)
    dtr = col(inp.dt_tok) if args.dt_shared else col(inp.dt_raw)
    z = col(inp.z) if w.gate else None
    dtb, A, Dk = t32(inp.dt_bias), t32(inp.A), t32(inp.Dskip)
    h = t32(inp.h0)
    y = torch.empty((w.batch, w.dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        ss.ss_step(x, dtr, dtb, A, Bm, Cm, Dk, h, z=z, y=y, disc=args.disc, stream=stream)

    if args.graph:
        return run_decode_graph(args, w, step_graphable=lambda s: ss.ss_step(
            x, dtr, dtb, A, Bm, Cm, Dk, h, z=z, y=y, disc=args.disc, stream=s))
    # the state (B*D*N*4 bytes) fits in the 256 MB Infinity Cache: an untimed 1 GiB write
    # between steps evicts it, so each timed step reads and writes HBM
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calib_copy(args, dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in evs:
        if flush is not None:
            flush.fill_(1)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e-3
    t_avg = float(per.mean())
    s_in = 2 if w.dtype == "bf16" else 4
    mb = step_min_bytes(w, s_in, args.dt_shared)
    gbps = mb / t_avg / 1e9
    elems = w.batch * w.dim
    log(f"[bench] decode step event avg {t_avg * 1e6:.2f} us (min {per.min() * 1e6:.2f}); "
        f"{mb / 1e6:.1f} MB min bytes -> {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.3f} of 8 TB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, disc=args.disc)
        log(f"[bench] cpu baseline {cpu['value']:.3e} elem/s ({cpu['sample']})")
    out = {
        "metric": "selective-scan decode step B·D channel-steps/s; achieved HBM GB/s vs MI355X peak",
        # with flushes between steps the wall clock includes them: value and ms_per_step
        # come from the HIP events around each step
        "value": elems / t_avg, "unit": "elem/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_avg * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.label}", "batch": w.batch, "seqlen": 1,
                   "dim": w.dim, "dstate": w.dstate, "in_dtype": w.dtype, "gate": w.gate,
                   "cache_flush_mib": args.flush_mib,
                   "disc": "zoh" if args.disc else "first-order"},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": None if args.dt_shared else measured_traffic(w, args.disc),
                     "kernel": "ss_step (step_kernel, one launch per call)",
                     "launch_us": t_avg * 1e6, "traffic_algorithmic_bytes": mb},
        "cpu_baseline": cpu,
    }
    emit(out)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def block_cpu_baseline(w, inp, budget_s=4.0):
    """The fp64 block oracle (numpy projections, C scan) timed on a growing prefix of the
    first batch row's tokens until one run takes about budget_s seconds."""
    from oracle import block_ref, cref
    threads = cref.threads(0)
    n = 16
    while True:
        t0 = time.perf_counter()
        block_ref.block_fwd(inp.u[:1, :n], inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip,
                            impl="c")
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n >= w.seqlen:
            break
        n = min(w.seqlen, int(n * max(2.0, budget_s / max(dt, 1e-3) / 2)))
    elems = n * w.dim
    return {"value": elems / dt, "unit": "elem/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batch row 0, first {n} of {w.seqlen} tokens, all {w.dim} channels "
                      f"(B*L*D elements {elems}), {dt:.2f} s wall; numpy float64 matrix products "
                      f"and the C scan on {threads} OpenMP threads"}


def run_block(args, w, inp):
    """Block workload: K timed ss_block_fwd calls (input projection on the matrix cores,
    selection projections, gated scan); then K ss_in_proj calls timed alone, the dominant
    kernel, for the MFMA roofline."""
    import torch
    import selective_state_space_34_amd as ss
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    u, W_in = bf(inp.u), bf(inp.W_in)
    W_x, dtb, A, Dk = f32(inp.W_x), f32(inp.dt_bias), f32(inp.A), f32(inp.Dskip)
    y = torch.empty((w.batch, w.seqlen, w.dim), dtype=torch.float32, device=dev)
    dims = ss.make_block_dims(w.batch, w.seqlen, w.d_in, w.dim, w.dstate)
    ws = torch.empty(ss.block_workspace_size(dims), dtype=torch.uint8, device=dev)
    xo = torch.empty((w.batch, w.seqlen, w.dim), dtype=torch.float32, device=dev)
    zo = torch.empty_like(xo)
    stream = torch.cuda.current_stream()

    def step():
        ss.ss_block_fwd(u, W_in, W_x, dtb, A, Dk, y=y, workspace=ws, stream=stream)

    def gemm():
        ss.ss_in_proj(u, W_in, x=xo, z=zo, stream=stream)

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e-3, wall

    for _ in range(args.warmup):
        step()
        gemm()
    torch.cuda.synchronize()
    calib_copy(args, dev)
    per, wall = timed(step)
    gper, _ = timed(gemm)
    t_avg, tg = float(per.mean()), float(gper.mean())
    vendor = None
    if args.vendor_gemm:
        # the same product by the vendor GEMM torch.matmul calls (bf16 result: torch has no
        # bf16 x bf16 -> float32 product), a reference point for the projection kernel only
        u2, Wt = u.reshape(-1, w.d_in), W_in.t()
        o16 = torch.empty((u2.shape[0], 2 * w.dim), dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup):
            torch.matmul(u2, Wt, out=o16)
        vper, _ = timed(lambda: torch.matmul(u2, Wt, out=o16))
        vendor = float(vper.mean())
    M = w.batch * w.seqlen
    flops = 2.0 * M * (2 * w.dim) * w.d_in
    tflops = flops / tg / 1e12
    elems = M * w.dim
    log(f"[bench] block step event avg {t_avg * 1e6:.1f} us; input projection alone "
        f"{tg * 1e6:.1f} us = {tflops:.0f} TFLOP/s ({tflops / MFMA_BF16_PEAK_TFLOPS:.3f} of "
        f"{MFMA_BF16_PEAK_TFLOPS:.0f}); the rest {(t_avg - tg) * 1e6:.1f} us")
    if vendor is not None:
        log(f"[bench] vendor GEMM (torch.matmul, bf16 result) on the same product: "
            f"{vendor * 1e6:.1f} us = {flops / vendor / 1e12:.0f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = block_cpu_baseline(w, inp)
        log(f"[bench] cpu baseline {cpu['value']:.3e} elem/s ({cpu['sample']})")
    out = {
        "metric": "selective-scan block fwd B·L·D elements/s; input projection TFLOP/s vs "
                  "MI355X bf16 matrix peak",
        "value": elems * args.steps / wall, "unit": "elem/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x bf16 -> f32 (projection), f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.label}", "batch": w.batch, "seqlen": w.seqlen,
                   "d_in": w.d_in, "dim": w.dim, "dstate": w.dstate},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None,
                     "kernel": "gemm_bf16_nt_kernel (ss_in_proj, the block's input projection)",
                     "launch_us": tg * 1e6, "flops": flops},
        "block_split": {"step_us": t_avg * 1e6, "in_proj_us": tg * 1e6,
                        "rest_us": (t_avg - tg) * 1e6},
        "vendor_gemm_bf16_out_us": None if vendor is None else vendor * 1e6,
        "cpu_baseline": cpu,
    }
    emit(out)


def run_decode_graph(args, w, step_graphable):
    """Decode as a serving loop: `steps` consecutive ss_step calls captured in one HIP graph
    and replayed; the state stays warm between steps, as it does between tokens."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            step_graphable(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(args.steps):
            step_graphable(s)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = e0.elapsed_time(e1) * 1e-3 / (reps * args.steps)
    s_in = 2 if w.dtype == "bf16" else 4
    mb = step_min_bytes(w, s_in, args.dt_shared)
    gbps = mb / t_step / 1e9
    elems = w.batch * w.dim
    log(f"[bench] decode loop in one graph: {args.steps} steps x {reps} replays, "
        f"{t_step * 1e6:.2f} us per step; {gbps:.0f} GB/s of minimum bytes (state warm)")
    out = {
        "metric": "selective-scan decode step B·D channel-steps/s (graph-replayed loop, state warm)",
        "value": elems / t_step, "unit": "elem/s", "n_gpus": 1, "steps": args.steps * reps,
        "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.label}", "batch": w.batch, "seqlen": 1,
                   "dim": w.dim, "dstate": w.dstate, "in_dtype": w.dtype, "gate": w.gate,
                   "graph": True, "cache_flush_mib": 0,
                   "disc": "zoh" if args.disc else "first-order",
                   "wall_s": wall},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "ss_step (step_kernel, graph replay)",
                     "launch_us": t_step * 1e6, "traffic_algorithmic_bytes": mb},
        "cpu_baseline": None,
    }
    emit(out)


def calib_copy(args, dev):
    """One device copy of a known size, for scaling the HBM byte counters."""
    import torch
    if not args.calib_copy_mib:
        return
    nb = args.calib_copy_mib << 20
    a = torch.empty(nb, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {nb} bytes done")


def dims_plan_single(ss, dims):
    """True when the forward runs as one kernel launch (no chunk workspace)."""
    return ss.workspace_size(dims) == 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2",
                    help="c0..c4 (default c2, D=5120 forward); d1 = decode step; p2 = block")
    ap.add_argument("--plan", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunk length of the chunked forward plan (0 = the plan's choice)")
    ap.add_argument("--layout", type=int, default=0, help="0 auto, 1 four lanes, 2 one lane, 3 eight lanes per channel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--order", type=int, default=0,
                    help="0 channel-major [B,D,L] sequences, 1 token-major [B,L,D] (B, C [B,L,N])")
    ap.add_argument("--dt-shared", action="store_true",
                    help="one dt_raw value per token [B, L], shared by the channels")
    ap.add_argument("--disc", type=int, default=0,
                    help="0 first-order input term (δ·B·x), 1 exact zero-order hold (forward only)")
    ap.add_argument("--no-ckpt", action="store_true",
                    help="fwd+bwd: recompute chunk start states instead of using checkpoints")
    ap.add_argument("--graph", action="store_true",
                    help="decode: capture the timed steps in one HIP graph and replay it")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="decode, and forwards under 512 MB: untimed write of this many MiB "
                         "before each timed step (0 = none)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="block workload: also time the vendor GEMM (torch.matmul) on the input "
                         "projection's product, for reference")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also launch one device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward would shard by batch or channel with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_34_amd as ss
    from gen import workload, workload_inputs

    w = workload(args.workload)
    log(f"[bench] workload {w.name}: {w.label}")
    t0 = time.perf_counter()
    inp = workload_inputs(w) if w.d_in else workload_inputs(w, dt_shared=args.dt_shared)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    if w.decode:
        run_decode(args, w, inp)
        return
    if w.d_in:
        run_block(args, w, inp)
        return
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    # the same values in the requested memory order
    lay = (lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))) if args.order else (lambda a: a)
    t_in = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    t32 = lambda a: torch.from_numpy(a).to(dev)
    x, Bm, Cm = t_in(lay(inp.x)), t_in(lay(inp.Bm)), t_in(lay(inp.Cm))
    dtr = t_in(inp.dt_tok) if args.dt_shared else t_in(lay(inp.dt_raw))
    z = t_in(lay(inp.z)) if w.gate else None
    dtb, A, Dk = t32(inp.dt_bias), t32(inp.A), t32(inp.Dskip)
    yshape = (w.batch, w.seqlen, w.dim) if args.order else (w.batch, w.dim, w.seqlen)
    y = torch.empty(yshape, dtype=torch.float32, device=dev)
    hf = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev) if w.h_final else None
    dims = ss.make_dims(w.batch, w.seqlen, w.dim, w.dstate,
                        ss.SS_BF16 if w.dtype == "bf16" else ss.SS_F32, args.plan, args.chunk, args.layout,
                        args.disc, args.order,
                        ss.SS_DT_SHARED if args.dt_shared else ss.SS_DT_FULL)
    ws = torch.empty(max(ss.workspace_size(dims), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    hck = None
    if w.backward:
        dy = t32(np.ascontiguousarray(lay(inp.dy)))
        # the backward keeps its own chunk length (--chunk sets the forward's)
        bdims = ss.make_dims(w.batch, w.seqlen, w.dim, w.dstate,
                             ss.SS_BF16 if w.dtype == "bf16" else ss.SS_F32, 0, 0, 0, args.disc,
                             args.order, ss.SS_DT_SHARED if args.dt_shared else ss.SS_DT_FULL)
        wsb = torch.empty(ss.workspace_size(bdims, backward=True), dtype=torch.uint8, device=dev)
        grads = ss.ss_bwd(x, dtr, dtb, A, Bm, Cm, Dk, dy, z=z, order=args.order, disc=args.disc)
        # training use: the forward keeps its 16-step state checkpoints for the backward
        if not args.no_ckpt:
            nck = (w.seqlen + ss.CKPT_STEPS - 1) // ss.CKPT_STEPS
            hck = torch.empty((w.batch, w.dim, nck, w.dstate), dtype=torch.float32, device=dev)

    def fwd_call():
        ss.ss_fwd(x, dtr, dtb, A, Bm, Cm, Dk, z=z, y=y, h_final=hf, h_ckpt=hck, workspace=ws,
                  plan=args.plan, chunk=args.chunk, layout=args.layout, disc=args.disc,
                  order=args.order, stream=stream)

    def bwd_call():
        ss.ss_bwd(x, dtr, dtb, A, Bm, Cm, Dk, dy, z=z, h_ckpt=hck, workspace=wsb, out=grads,
                  order=args.order, disc=args.disc, stream=stream)

    def step():
        fwd_call()
        if w.backward:
            bwd_call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calib_copy(args, dev)

    # A forward whose bytes fit in the 256 MB Infinity Cache would be timed warm: an untimed
    # 1 GiB write before each timed step evicts it, and the step is then timed by its events.
    s_in0 = 2 if w.dtype == "bf16" else 4
    cold = (not w.backward and args.flush_mib > 0
            and min_bytes(w, s_in0, args.dt_shared) < (512 << 20))
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if cold else None

    # timed region: K steps, HIP events around every step on the stream the kernels run on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in evs:
        if flush is not None:
            flush.fill_(1)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e-3  # seconds per step
    if flush is not None:
        wall = float(per.sum())   # the flushes are outside the events
    split = None
    if w.backward:
        # the forward alone, timed the same way, so the backward's share is known
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in fe:
            e0.record(stream)
            fwd_call()
            e1.record(stream)
        torch.cuda.synchronize()
        tf = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fe])) * 1e-3
        split = {"fwd_us": tf * 1e6, "bwd_us": (float(per.mean()) - tf) * 1e6,
                 "bwd_min_bytes": bwd_min_bytes(w, 2 if w.dtype == "bf16" else 4, args.dt_shared)}
        log(f"[bench] fwd {tf * 1e6:.1f} us, bwd {(float(per.mean()) - tf) * 1e6:.1f} us "
            f"(bwd min bytes {split['bwd_min_bytes'] / 1e6:.1f} MB -> "
            f"{split['bwd_min_bytes'] / (float(per.mean()) - tf) / 1e9:.0f} GB/s)")

    elems = w.batch * w.seqlen * w.dim
    s_in = 2 if w.dtype == "bf16" else 4
    mb = min_bytes(w, s_in, args.dt_shared)
    t_avg = float(per.mean())
    value = elems * args.steps / wall
    slots_pe = alu_slots_per_elem(w, args.disc) + (bwd_alu_slots_per_elem(w, args.disc)
                                                    if w.backward else 0)
    slots = elems * slots_pe
    alu_achieved = slots / t_avg / 1e12
    hbm_achieved = mb / t_avg / 1e9
    log(f"[bench] per-step event time avg {t_avg * 1e6:.1f} us (min {per.min() * 1e6:.1f}, "
        f"max {per.max() * 1e6:.1f}); wall {wall / args.steps * 1e6:.1f} us/step")
    log(f"[bench] HBM view: {mb / 1e6:.1f} MB min bytes -> {hbm_achieved:.0f} GB/s "
        f"({hbm_achieved / HBM_PEAK_GBPS:.3f} of 8 TB/s)")
    log(f"[bench] ALU view: {slots_pe} slots/elem -> {alu_achieved:.2f} T slots/s "
        f"({alu_achieved / ALU_PEAK_TSLOTS:.3f} of {ALU_PEAK_TSLOTS:.2f})")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline ...")
        cpu = cpu_baseline(w, inp, disc=args.disc)
        log(f"[bench] cpu baseline {cpu['value']:.3e} elem/s ({cpu['sample']})")

    out = {
        "metric": "selective-scan fwd B·L·D elements/s; achieved HBM GB/s vs MI355X peak",
        "value": value,
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.label}", "batch": w.batch, "seqlen": w.seqlen,
                   "dim": w.dim, "dstate": w.dstate, "in_dtype": w.dtype, "gate": w.gate,
                   "plan": args.plan, "chunk": args.chunk, "layout": args.layout,
                   "disc": "zoh" if args.disc else "first-order",
                   "cache_flush_mib": args.flush_mib if flush is not None else 0,
                   "order": "BLD" if args.order else "BDL",
                   "dt_raw": "shared [B,L]" if args.dt_shared else "per channel",
                   "checkpoints": bool(w.backward and not args.no_ckpt)},
        "roofline": {"bound": "alu", "achieved": alu_achieved, "peak": ALU_PEAK_TSLOTS,
                     "unit": "T VALU-slot/s", "frac": alu_achieved / ALU_PEAK_TSLOTS,
                     "traffic": (None if args.order or args.dt_shared
                                 else measured_traffic(w, args.disc)),
                     "kernel": ("ss_fwd + ss_bwd step (every kernel of both calls)" if w.backward
                                else "ss_fwd (one group-scan launch per call: scang_kernel, or "
                                     "scang_mixed_kernel for the four/eight-lane mixed layout)"
                                if dims_plan_single(ss, dims) else "ss_fwd (all passes)"),
                     "launch_us": t_avg * 1e6, "launch_us_median": float(np.median(per)) * 1e6,
                     "slots_per_elem": slots_pe,
                     "traffic_algorithmic_bytes": mb if not w.backward else None},
        "hbm": {"min_bytes": mb, "achieved_gbps": hbm_achieved, "peak_gbps": HBM_PEAK_GBPS,
                "frac": hbm_achieved / HBM_PEAK_GBPS},
        "cpu_baseline": cpu,
    }
    if split:
        out["fwd_bwd_split"] = split
    emit(out)


if __name__ == "__main__":
    main()
