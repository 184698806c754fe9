"""Benchmark of one hybrid Muon + AdamW optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]

A step is the whole hot path over one batch of synthetic gradients already resident
in HBM: ma_adamw_step over the flat AdamW buffer, then ma_muon_step over every shape
bucket (momentum, normalisation, 5 Newton-Schulz iterations, update), all on one
stream.  Printed: one JSON line with the step time (ms), the Newton-Schulz GEMM
throughput against the bf16 MFMA peak and the AdamW bandwidth against HBM peak, each
measured with HIP events on the launch stream, plus the fp64 CPU oracle timed on a
bounded sample of the same workload.

Default workload: index 4, one GPU's owned subset at large shape (8 x 8192x28672,
8 x 28672x8192 and 16 x 8192x8192 Muon matrices, a 128256x8192 AdamW embedding), the
largest configuration that fits one GPU; --workload 0-3 select the smaller ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
ADAMW_BYTES_PER_ELEM = 28        # read p, g, m, v; write p, m, v (fp32)


def gram_space(b, ns_mode):
    """Whether the library runs this bucket's Newton-Schulz in Gram space (its own
    routing report: buckets whose long side is at least 3x the Gram side, under ns_mode 1)."""
    if ns_mode != 1:
        return False
    import adamw_optimizer_step_muon_amd as ma

    return bool(ma.muon_route_of(b.A, b.B, 5, ns_mode=1).ns_mode_run)


def ns_flops(wl, steps=None, symmetric=True, ns_mode=0):
    """Algorithmic Newton-Schulz FLOP of one optimizer step.  Printed iteration, per matrix
    and iteration: 3 m^2 n + m^3 with the symmetric Gram and R R^T on one triangle (dense:
    4 m^2 n + 2 m^3).  Gram-space route (ns_mode 1, n >= 3 m), per matrix for N steps:
    the Gram m^2 n, N polynomials, N - 1 products P Q, 2 (N - 1) products for R <- P R P
    (m^3 each on one triangle), and the final Q X0, 2 m^2 n: 3 m^2 n + (4 N - 3) m^3
    (dense: 4 m^2 n + (8 N - 6) m^3)."""
    N = wl.muon_hp.ns_steps if steps is None else steps
    total = 0
    for b in wl.muon:
        m, n = min(b.A, b.B), max(b.A, b.B)
        if gram_space(b, ns_mode) and N > 0:
            per = (3 * m * m * n + (4 * N - 3) * m ** 3) if symmetric else (
                4 * m * m * n + (8 * N - 6) * m ** 3)
        else:
            per = N * ((3 * m * m * n + m ** 3) if symmetric else (4 * m * m * n + 2 * m ** 3))
        total += b.K * per
    return total


def ns_bytes(wl, ns_mode=0):
    """Algorithmic HBM bytes of the Newton-Schulz launches of one step (16-bit operands and
    results, each read or written once, padding ignored).  Printed iteration, per matrix
    and iteration: the Gram reads X and writes R (m n + m^2), the polynomial reads R and
    writes P (2 m^2), the combine reads P and X and writes X' (m^2 + 2 m n): 2 (3 m n +
    4 m^2) bytes.  Gram-space route: the Gram (m n + m^2), per step a polynomial (2 m^2),
    then 3 m^2 per symmetric product (two operands, one result) for the 3 (N - 1)
    products, and the final product (m^2 + 2 m n)."""
    N = wl.muon_hp.ns_steps
    total = 0
    for b in wl.muon:
        m, n = min(b.A, b.B), max(b.A, b.B)
        if gram_space(b, ns_mode) and N > 0:
            per = (m * n + m * m) + N * 2 * m * m + 3 * (N - 1) * 3 * m * m + (m * m + 2 * m * n)
        else:
            per = N * (3 * m * n + 4 * m * m)
        total += 2 * b.K * per
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ns-mode", type=int, default=0, choices=(0, 1),
                    help="1: the fp16 Gram-space Newton-Schulz for buckets whose long side is "
                         "at least 3.5x the Gram side (opt-in; by default it is timed beside "
                         "the printed iteration and reported as gram_space_route)")
    ap.add_argument("--no-tune", action="store_true",
                    help="keep the default GEMM rules instead of searching each Newton-Schulz "
                         "product's configuration once before the warm-up "
                         "(ma_muon_tune_configs)")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, copy this many MiB device-to-device once (a plain "
                         "copy of known size for calibrating HBM byte counters)")
    ap.add_argument("--no-alt-route", action="store_true",
                    help="skip timing the opt-in fp16 Gram-space route (ns_mode 1) beside the "
                         "printed iteration")
    ap.add_argument("--comparator", action="store_true",
                    help="also time the same Newton-Schulz chain as torch bf16 batched GEMMs "
                         "(hipBLASLt) on the workload's gradients, after the measurement")
    ap.add_argument("--zero-operands", action="store_true",
                    help="also time the Newton-Schulz launches on zero gradients: operands "
                         "that do not toggle take the power limit out, so the rate shows "
                         "what the kernels' structure allows at the full clock")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "adamw_optimizer_step_muon_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_hash(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


ns_mode_of_run = 0  # set by main: the committed summaries profile the printed iteration


def counted_traffic(summary, source, key="traffic_bytes_per_launch"):
    """A figure (HBM bytes per launch by default) from a committed rocprofv3 counter
    summary, or None when the summary is missing or the kernel source changed since."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    vals = {}
    if ns_mode_of_run != 0:
        return None  # the summaries describe the default route's launches
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("source_sha256") != source_hash(source):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def oracle_cost(b):
    """Relative cost of the oracle on one A x B matrix: two m^2 n products (the Gram
    matrix and the final product) and the symmetric eigendecomposition of the m x m
    Gram matrix, which on the host costs about as much as 10 m^3 of matrix products
    (measured: 8192 x 8192 and 8192 x 28672 in 46 and 78 s on 8 cores)."""
    m, n = min(b.A, b.B), max(b.A, b.B)
    return 4 * m * m * n + 10 * m ** 3


def cpu_baseline(wl, budget_s):
    """The fp64 oracle as it stands on the host cores, timed on a bounded sample of one
    step and scaled to the whole step.  About budget_s seconds of oracle work: half on
    Muon matrices, taken round-robin over the buckets from the cheapest bucket up
    (matrix k of every bucket before matrix k + 1 of any), half on AdamW slices of 4M
    elements.  Each bucket's time is its mean per sampled matrix x K; a bucket the
    budget never reached is extrapolated from the sampled ones by the oracle's cost
    model (oracle_cost), and the sample text says so.  Input generation is not timed."""
    import numpy as np

    import oracle
    from workloads import gen

    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    hp = wl.muon_hp
    nb = len(wl.muon)
    per_t, per_n = [0.0] * nb, [0] * nb
    by_cost = sorted(range(nb), key=lambda bi: oracle_cost(wl.muon[bi]))
    order = [(bi, k) for k in range(max(b.K for b in wl.muon)) for bi in by_cost
             if k < wl.muon[bi].K]
    t_muon = 0.0
    for bi, k in order:
        if per_n != [0] * nb and t_muon >= budget_s / 2:
            break
        b = wl.muon[bi]
        p0 = gen.np_param(wl.seed, gen.muon_index(wl, bi, k), (b.A, b.B))
        g1 = gen.np_grad(wl.seed, 1, gen.muon_index(wl, bi, k), (b.A, b.B), wl.muon_grad,
                         wl.muon_sigma)
        t0 = time.perf_counter()
        oracle.muon_step(p0, g1, np.zeros((b.A, b.B)), lr=hp.lr, mu=hp.momentum,
                         weight_decay=hp.weight_decay, cautious_wd=hp.cautious_wd)
        dt = time.perf_counter() - t0
        per_t[bi] += dt
        per_n[bi] += 1
        t_muon += dt

    s_per_unit = sum(per_t) / sum(oracle_cost(b) * per_n[i] for i, b in enumerate(wl.muon))
    muon_s = 0.0
    parts = []
    for bi, b in enumerate(wl.muon):
        if per_n[bi]:
            muon_s += per_t[bi] / per_n[bi] * b.K
            parts.append(f"{per_n[bi]} of {b.K} {b.A}x{b.B}")
        else:
            muon_s += s_per_unit * oracle_cost(b) * b.K
            parts.append(f"0 of {b.K} {b.A}x{b.B} (extrapolated by the oracle's cost model "
                         "4 m^2 n + 10 m^3)")
    n = wl.adamw_numel
    ah = wl.adamw_hp
    chunk = min(n, 4_000_000)
    rng = np.random.default_rng(0)
    t_adamw, n_done = 0.0, 0
    while n_done < n and (n_done == 0 or t_adamw < budget_s / 2):
        c = min(chunk, n - n_done)
        p = rng.standard_normal(c).astype(np.float32)
        g = (1e-3 * rng.standard_normal(c)).astype(np.float32)
        t0 = time.perf_counter()
        oracle.adamw_step(p, g, np.zeros(c), np.zeros(c), step=1, lr=ah.lr, beta1=ah.beta1,
                          beta2=ah.beta2, eps=ah.eps, weight_decay=ah.weight_decay)
        t_adamw += time.perf_counter() - t0
        n_done += c
    adamw_s = t_adamw * (n / n_done)
    return {"value": round((muon_s + adamw_s) * 1e3, 1), "unit": "ms", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"one step, {t_muon + t_adamw:.1f} s of oracle work: Muon {', '.join(parts)} "
                       f"matrices, each bucket scaled by K; AdamW {n_done} of {n} elements, "
                       f"scaled; numpy float64 (BLAS threads={cores}, elementwise "
                       "single-threaded)")}


def alt_route(wl, buckets, state, adamw, stream, dev, args):
    """The same step with the opt-in fp16 Gram-space route (ns_mode 1) for the buckets it
    takes, timed after the headline measurement on the same state: its configuration
    search, one warm-up step, then min(steps, 5) steps between HIP events, and its
    Newton-Schulz launches per phase (ma_muon_ns_time)."""
    import torch

    import adamw_optimizer_step_muon_amd as ma

    mh = wl.muon_hp
    shapes = [(b.K, b.A, b.B) for b in wl.muon]
    ws = torch.empty(max(ma.muon_workspace_bytes(shapes, 1), 1), dtype=torch.uint8, device=dev)
    if not args.no_tune:
        ma.muon_tune_configs(shapes, reps=3, workspace=ws, stream=stream, ns_mode=1,
                             grads=[b[1] for b in buckets])
    routes = []

    def step():
        state["t"] += 1
        adamw()
        routes[:] = ma.muon_step(buckets, lr=mh.lr, momentum=mh.momentum,
                                 weight_decay=mh.weight_decay, nesterov=mh.nesterov,
                                 ns_steps=mh.ns_steps, ns_eps=mh.ns_eps,
                                 cautious_wd=mh.cautious_wd, scale_mode=mh.scale_mode,
                                 ns_mode=1, workspace=ws, stream=stream)

    step()
    k = max(1, min(args.steps, 5))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(k):
        step()
    e1.record(stream)
    e1.synchronize()
    step_ms = e0.elapsed_time(e1) / k
    phase_ms = ma.muon_ns_time([b[1] for b in buckets], reps=3, ns_steps=mh.ns_steps,
                               ns_eps=mh.ns_eps, ns_mode=1, workspace=ws, stream=stream)
    del ws
    torch.cuda.empty_cache()
    return {"ns_mode": 1, "operands": "fp16 (Gram-space products), bf16 result",
            "buckets_on_route": [int(r.ns_mode_run) for r in routes], "steps": k,
            "step_ms": round(step_ms, 4), "ns_ms": round(sum(phase_ms), 4),
            "ns_phase_ms": [round(x, 4) for x in phase_ms],
            "ns_tflops_algorithmic": round(ns_flops(wl, ns_mode=1) / (sum(phase_ms) * 1e-3) / 1e12, 1),
            # the printed iteration's FLOP count over this route's time: the rate a printed
            # iteration would need to match it (context for the saving, not a kernel rate)
            "ns_tflops_printed_equivalent": round(ns_flops(wl, ns_mode=0) / (sum(phase_ms) * 1e-3) / 1e12, 1)}


def blas_comparator(grads, coeffs, ns_steps, stream, reps=3):
    """The Newton-Schulz chain of each bucket as plain torch bf16 batched GEMMs (hipBLASLt
    on this image): X = G / ||G||_F per matrix in bf16, wide orientation; per step
    R = X X^T, P = b R + c R R, X = a X + P X (bmm / baddbmm, both operands contiguous).
    Timed with HIP events on the launch stream; the normalisation and cast stay outside."""
    import torch

    a, b, c = coeffs
    total_ms, sym, dense, per = 0.0, 0.0, 0.0, []
    for g in grads:
        K, A, B = g.shape
        m, n = min(A, B), max(A, B)
        X0 = g if A <= B else g.mT
        X0 = (X0 / X0.norm(dim=(1, 2), keepdim=True).clamp_min(1e-30)).to(torch.bfloat16).contiguous()

        def chain():
            X = X0
            for _ in range(ns_steps):
                R = torch.bmm(X, X.mT.contiguous())
                P = torch.baddbmm(R, R, R, beta=b, alpha=c)
                X = torch.baddbmm(X, P, X, beta=a, alpha=1.0)
            return X

        chain()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            chain()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        total_ms += ms
        sym += K * ns_steps * (3 * m * m * n + m ** 3)
        dense += K * ns_steps * (4 * m * m * n + 2 * m ** 3)
        per.append(round(ms, 4))
        del X0
        torch.cuda.empty_cache()
    return {"kind": "torch bf16 bmm/baddbmm chain (hipBLASLt), same buckets and data",
            "ns_ms": round(total_ms, 4), "bucket_ms": per,
            "tflops_symmetric_count": round(sym / (total_ms * 1e-3) / 1e12, 1),
            "tflops_dense_count": round(dense / (total_ms * 1e-3) / 1e12, 1)}


def mfma_probe(grad, dev, stream, iters=300000, reps=3):
    """Sustained bf16 MFMA rate and shader clock of ma_mfma_probe over the whole chip: once
    on the first 8192 values of a Muon gradient (cast to bf16; the GEMMs' operands are
    such values scaled), once on zeros.  TFLOP/s from HIP events on the launch stream,
    the clock from the probe's own cycle counters."""
    import torch

    import adamw_optimizer_step_muon_amd as ma

    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(blocks * ma.MFMA_PROBE_THREADS, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    vals = grad.reshape(-1)[:ma.MFMA_PROBE_OPERAND_VALUES].to(torch.bfloat16).contiguous()
    res = {}
    for name, ops in (("", vals), ("_zero_operands", torch.zeros_like(vals))):
        ma.mfma_probe(ops, out, iters, clocks=clocks, stream=stream)   # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            ma.mfma_probe(ops, out, iters, clocks=clocks, stream=stream)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        c = clocks.double().cpu()
        res["tflops" + name] = round(ma.mfma_probe_flops(blocks, iters) / (ms * 1e-3) / 1e12, 1)
        res["clock_ghz" + name] = round(float(c[0::2].sum() / c[1::2].sum()) * 0.1, 3)
    res["operands"] = "first 8192 values of the first Muon bucket's gradient, as bf16"
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(each owner's share runs on its own GPU, see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    import adamw_optimizer_step_muon_amd as ma
    import workloads
    from workloads import gen

    global ns_mode_of_run
    ns_mode_of_run = args.ns_mode
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.workload(args.workload)
    mh, ah = wl.muon_hp, wl.adamw_hp

    # ---- inputs resident in HBM ----
    buckets = []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=dev)
        g = torch.empty_like(p)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        gen.torch_muon_bucket(torch, wl, bi, 1, g)
        buckets.append((p, g, torch.zeros_like(p)))
    n = wl.adamw_numel
    ap_ = torch.empty(n, dtype=torch.float32, device=dev)
    ag = torch.empty_like(ap_)
    gen.torch_adamw_flat(torch, wl, 0, ap_)
    gen.torch_adamw_flat(torch, wl, 1, ag)
    am, av = torch.zeros_like(ap_), torch.zeros_like(ap_)
    ws = torch.empty(max(ma.muon_workspace_bytes([tuple(b[0].shape) for b in buckets],
                                                 args.ns_mode), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    state = {"t": 0}
    shapes = [(b.K, b.A, b.B) for b in wl.muon]
    # per-shape GEMM configurations (tile, pipeline, band width, spreading), searched once
    # on the workspace (untimed set-up, like the warm-up)
    ns_configs = (None if args.no_tune
                  else ma.muon_tune_configs(shapes, reps=3, workspace=ws, stream=stream,
                                            ns_mode=args.ns_mode, grads=[b[1] for b in buckets]))

    def adamw():
        ma.adamw_step(ap_, ag, am, av, step=state["t"], lr=ah.lr, beta1=ah.beta1, beta2=ah.beta2,
                      eps=ah.eps, weight_decay=ah.weight_decay, decoupled=ah.decoupled,
                      cautious_wd=ah.cautious_wd, stream=stream)

    def muon(ns_steps):
        ma.muon_step(buckets, lr=mh.lr, momentum=mh.momentum, weight_decay=mh.weight_decay,
                     nesterov=mh.nesterov, ns_steps=ns_steps, ns_eps=mh.ns_eps,
                     cautious_wd=mh.cautious_wd, scale_mode=mh.scale_mode, ns_mode=args.ns_mode,
                     workspace=ws, stream=stream)

    def step():
        state["t"] += 1
        adamw()
        muon(mh.ns_steps)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per call

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K steps between two synchronisations, one HIP event between
    # consecutive steps for the per-step median and minimum
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    step_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    median_ms = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])

    # ---- per-kernel figures, live, same stream ----
    reps = max(3, min(args.steps, 10))
    # the Newton-Schulz GEMM launches alone, per phase, between HIP events on the launch
    # stream (ma_muon_ns_time: each repetition casts the gradients first, untimed)
    phase_ms = ma.muon_ns_time([b[1] for b in buckets], reps=reps, ns_steps=mh.ns_steps,
                               ns_eps=mh.ns_eps, ns_mode=args.ns_mode, workspace=ws,
                               stream=stream)
    ns_ms = sum(phase_ms)
    muon_ms = timed(lambda: muon(mh.ns_steps), reps)
    # same-tile buckets share launches: 3 x ns_steps per phase of the printed iteration,
    # 4 ns_steps - 1 per Gram-space phase (Gram, polynomials, products, final product)
    phases, phase_of = ma.muon_phases(shapes, args.ns_mode)
    N = mh.ns_steps
    launches = 0
    for ph in range(phases):
        b = wl.muon[phase_of.index(ph)]
        launches += (4 * N - 1) if (gram_space(b, args.ns_mode) and N > 0) else 3 * N
    flops = ns_flops(wl, ns_mode=args.ns_mode)
    nbytes = ns_bytes(wl, args.ns_mode)
    intensity = flops / nbytes
    attainable = min(MFMA_BF16_PEAK_TFLOPS, intensity * HBM_PEAK_GBS / 1e3)
    ns_tflops = flops / (ns_ms * 1e-3) / 1e12
    state["t"] = 1
    adamw_ms = timed(adamw, reps)
    adamw_gbs = ADAMW_BYTES_PER_ELEM * n / (adamw_ms * 1e-3) / 1e9
    clock = counted_traffic(f"ns_gemm_mfma_workload{args.workload}.txt", "ns_gemm.hip",
                            key="clock_ghz")
    # the ceiling of AdamW's access pattern on this part: the same 4-read / 3-write stream
    # in place over the same buffers, with the same accesses and no arithmetic (last:
    # it overwrites the AdamW state)
    probe_ms = timed(lambda: ma.stream_probe([ap_, ag, am, av], [ap_, am, av], stream=stream),
                     reps)
    probe_gbs = ADAMW_BYTES_PER_ELEM * n / (probe_ms * 1e-3) / 1e9
    # the matrix cores' sustained rate on this workload's values (ma_mfma_probe: the GEMM
    # kernel's MFMA and occupancy, operands in registers, no memory traffic), and on zeros
    mfma_ceiling = mfma_probe(buckets[0][1], dev, stream)

    out = {
        "metric": "optimizer-step ms + NS TFLOP/s (%MFMA peak) + AdamW GB/s (%HBM)",
        "value": round(step_ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "bf16 MFMA operands, fp32 accumulation; fp32 elementwise state",
        "data": "synthetic (seeded device-generated gradients and N(0,1) parameters)",
        "config": {"workload": wl.name, "muon_buckets": [[b.K, b.A, b.B] for b in wl.muon],
                   "adamw_elements": n, "ns_steps": mh.ns_steps, "ns_mode": args.ns_mode,
                   "cautious_wd": mh.cautious_wd},
        "ns_configs": ns_configs,
        "step_ms_median": round(median_ms, 4),
        "step_ms_min": round(per_step[0], 4),
        "ns_tflops": round(ns_tflops, 2),
        "ns_mfma_frac": round(ns_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "ns_ms": round(ns_ms, 4),
        "ns_phase_ms": [round(x, 4) for x in phase_ms],
        "muon_step_ms": round(muon_ms, 4),
        "adamw_ms": round(adamw_ms, 4),
        "adamw_gbs": round(adamw_gbs, 1),
        "adamw_hbm_frac": round(adamw_gbs / HBM_PEAK_GBS, 4),
        "muon_elementwise_ms": round(max(muon_ms - ns_ms, 0.0), 4),
        "roofline": {
            "kernel": "ns_gemm_kernel (gram, poly, combine launches of Newton-Schulz)",
            "bound": "mfma",
            "achieved": round(ns_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ns_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": counted_traffic(f"ns_gemm_traffic_workload{args.workload}.txt", "ns_gemm.hip"),
            # fraction of the kernel's cycles the matrix cores were busy (rocprofv3
            # SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE, at the clock the part ran)
            "mfma_busy_counter": counted_traffic(f"ns_gemm_mfma_workload{args.workload}.txt",
                                                 "ns_gemm.hip", key="mfma_busy"),
            # the shader clock the GEMM kernels ran at (rocprofv3 GRBM_GUI_ACTIVE per XCD
            # over the kernel's duration), and the bf16 peak at that clock
            "clock_ghz_counter": clock,
            "peak_at_clock": round(MFMA_BF16_PEAK_TFLOPS * clock / 2.4, 1) if clock else None,
            "frac_at_clock": round(ns_tflops / (MFMA_BF16_PEAK_TFLOPS * clock / 2.4), 4)
            if clock else None,
            "flops_per_launch": flops / launches,
            "avg_launch_ms": ns_ms / launches,
            # the same launches against both ceilings: algorithmic FLOP per algorithmic HBM
            # byte, and the roofline's attainable rate min(MFMA peak, intensity x HBM peak)
            "intensity_flop_per_byte": round(intensity, 1),
            "achieved_hbm_gbs": round(nbytes / (ns_ms * 1e-3) / 1e9, 1),
            "attainable_tflops": round(attainable, 1),
            "frac_of_attainable": round(ns_tflops / attainable, 4),
            # what a register-only MFMA loop sustains on the part with these operand values:
            # the clock falls under the power limit when the operands toggle
            "mfma_ceiling": mfma_ceiling,
            "frac_of_mfma_ceiling": round(ns_tflops / mfma_ceiling["tflops"], 4),
        },
        "adamw_roofline": {
            "kernel": "adamw_vec_kernel",
            "bound": "hbm",
            "achieved": round(adamw_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(adamw_gbs / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(f"adamw_traffic_workload{args.workload}.txt", "adamw.hip"),
            "bytes_per_launch": ADAMW_BYTES_PER_ELEM * n,
            # a 4-read / 3-write fp32 stream in place with AdamW's accesses and no
            # arithmetic (ma_stream_probe), timed here: the access pattern's own ceiling
            "stream_ceiling_gbs": round(probe_gbs, 1),
            "frac_of_stream_ceiling": round(adamw_gbs / probe_gbs, 4),
        },
        "timed_wall_s": round(wall_s, 3),
    }
    if args.calibration_copy_mib > 0:
        nbytes = args.calibration_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = nbytes
    if args.ns_mode == 0 and not args.no_alt_route and any(gram_space(b, 1) for b in wl.muon):
        out["gram_space_route"] = alt_route(wl, buckets, state, adamw, stream, dev, args)
    if args.zero_operands:
        zeros = [torch.zeros_like(b[1]) for b in buckets]
        zphase = ma.muon_ns_time(zeros, reps=reps, ns_steps=mh.ns_steps, ns_eps=mh.ns_eps,
                                 ns_mode=args.ns_mode, workspace=ws, stream=stream)
        del zeros
        zms = sum(zphase)
        out["zero_operands"] = {"ns_ms": round(zms, 4), "ns_tflops": round(flops / (zms * 1e-3) / 1e12, 1),
                                "ns_mfma_frac": round(flops / (zms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                "ns_phase_ms": [round(x, 4) for x in zphase]}
    if args.comparator:
        comp = blas_comparator([b[1] for b in buckets], mh.coeffs, mh.ns_steps, stream)
        comp["speedup_of_this_library"] = round(comp["ns_ms"] / ns_ms, 3)
        out["comparator"] = comp
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
