"""Benchmark of one Muon optimizer step on one MI355X.

A step is the whole hot path over every matrix of the workload:
momentum (fp32 momentum, Nesterov blend, sum of squares; it writes the
Newton-Schulz input) -> 5 quintic Newton-Schulz steps (bf16 MFMA with fp32
accumulation) -> the update (0.2*sqrt(max(m,n)) shape factor, decoupled
weight decay), with inputs resident in HBM.  By default the update is
applied by the last Newton-Schulz step (muon_momentum_packed_grouped, then
muon_orthogonalize_apply_packed_grouped); --separate-apply runs it as its own
kernel (muon_orthogonalize_packed_grouped, then muon_apply_grouped).

Prints one JSON line.  ``value`` is optimizer steps per second; the line
also carries the Newton-Schulz TFLOP/s (algorithmic flops: upper-triangle
Gram and square, full update product), the roofline of the dominant kernel
family and the fp64 CPU oracle timed on a bounded sample.

The default workload is the 32-layer dense set (224 matrices); the timed
region is exactly K steps enqueued back to back between two device
synchronizations, split by events into up to five blocks whose rates give
the median and spread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b-dense-32-layers]
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

METRIC = "Muon steps/sec + Newton-Schulz TFLOP/s (% bf16 MFMA peak) per layer set"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
LR, WD = 3e-4, 0.1


def ns_flops(count, rows, cols, steps=5):
    """(algorithmic, nominal) Newton-Schulz flops for `count` rows x cols."""
    m, n = min(rows, cols), max(rows, cols)
    algo = m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n
    nominal = 4 * m * m * n + 2 * m ** 3
    return count * steps * algo, count * steps * nominal


def momentum_bytes(cfg, packed):
    """Algorithmic bytes of the momentum phase: G (bf16) read, M (fp32) read
    and written, and the Newton-Schulz input written.  Unpacked, that input
    is N in fp32 (4 B per element).  Packed, it is written once into the
    padded Newton-Schulz buffers (tile 128 for a short side up to 128, else
    256): the bf16 high part (2 B) and the 8-bit residual with one exponent
    byte per 16 codes (1.0625 B); the bf16 update reads X itself, so no
    transposed copy is written."""
    def pad(x, t):
        return (x + t - 1) // t * t
    base = cfg.elements * (2 + 8)
    if not packed:
        return base + cfg.elements * 4
    out = base
    for g in cfg.groups:
        t = 128 if min(g.rows, g.cols) <= 128 else 256
        padded = pad(min(g.rows, g.cols), t) * pad(max(g.rows, g.cols), t)
        out += g.count * padded * (2 + 1.0625)
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Coefficient sets of the pages' Newton-Schulz iterations and their usual step counts: Jordan's quintic
# (5 steps), the convergent "Track-3" quintic (12 steps) and the classical cubic.
COEFFS = {"quintic": ((3.4445, -4.7750, 2.0315), 5), "track3": ((2.0, -1.5, 0.5), 12), "cubic": ((1.5, -0.5, 0.0), 5)}


def make_stepper(mx, weights, grads, coeffs="quintic", steps=None, fused_apply=True):
    """The optimizer step this benchmark times: every group of the workload
    in one MuonStep (grouped Newton-Schulz launches, bf16 MFMA; by default
    the update applied by the last Newton-Schulz step's epilogue)."""
    abc, k = COEFFS[coeffs]
    return mx.MuonStep(list(zip(weights, grads)), compute=mx.MUON_BF16, lr=LR, weight_decay=WD, coeffs=abc,
                       steps=k if steps is None else steps, fused_apply=fused_apply)


def ns_call(stepper):
    """The entry point that runs the Newton-Schulz steps of a MuonStep."""
    if stepper.packed and stepper.fused_apply:
        return "muon_orthogonalize_apply_packed_grouped"
    return "muon_orthogonalize_packed_grouped" if stepper.packed else "muon_orthogonalize_grouped"


def measured_traffic(profile, source, key):
    """HBM bytes per step from a rocprofv3 FETCH_SIZE/WRITE_SIZE summary in
    profiles/ (its traffic-record line), or None when the summary is missing
    or was taken on a different version of the kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "matrix_aware_optimizer_step_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
    if rec is None:
        return None
    if rec.get("kernel_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return rec[key]


ADAM_LR, ADAM_WD, ADAM_BETAS, ADAM_EPS = 3e-4, 0.1, (0.9, 0.999), 1e-8
ADAMW_BYTES = 2 + 2 + 2 + 8 + 8  # per element: bf16 theta read+write, bf16 grad, fp32 m and v read+write


def make_adamw_step(mx, names, params, grads):
    """The AdamW leg this benchmark times: the routing helper over the 8B-style
    model's non-matrix parameters (every one goes to AdamW)."""
    opt = mx.OptimizerStep(list(zip(names, params, grads)), adam_lr=ADAM_LR, adam_betas=ADAM_BETAS,
                           adam_eps=ADAM_EPS, adam_weight_decay=ADAM_WD)
    assert opt.muon is None
    return opt


def calibration_copy(dev):
    """One 1 GiB device-to-device copy, so that profiler byte counters can be
    scaled against a kernel of known traffic."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log("[bench] 1 GiB calibration copy done")


def bench_adamw(args):
    """Time the AdamW step over the 8B-style model's embeddings, head and norms;
    print one JSON line against the HBM roofline."""
    import numpy as np
    import torch

    import matrix_aware_optimizer_step_amd as mx
    from workloads import synth

    mx._lib.load()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    shapes = synth.adamw_workload()
    names = [n for n, _ in shapes]
    params, grads = synth.adamw_tensors(shapes, step=1, device=dev)
    opt = make_adamw_step(mx, names, params, grads)
    elems = sum(g.elements for g in opt.adamw)
    log(f"[bench] AdamW over {len(shapes)} tensors, {elems / 1e6:.1f} M elements")
    if args.copy_calibration:
        calibration_copy(dev)
    for _ in range(args.warmup):
        opt.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        opt.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    gbs = elems * ADAMW_BYTES / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import adamw as OA
        n = 1 << 24
        rng = np.random.default_rng(0)
        th, g = rng.standard_normal(n) * 0.02, rng.standard_normal(n)
        m, v = np.zeros(n), np.zeros(n)
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < 10.0:
            th, m, v = OA.adamw_step(th, g, m, v, reps + 1, ADAM_LR, *ADAM_BETAS, ADAM_EPS, ADAM_WD)
            reps += 1
        sec = (time.perf_counter() - t1) / reps * elems / n
        cpu = {"value": 1.0 / sec, "unit": "steps/s", "cores": 1, "kind": "oracle",
               "sample": f"fp64 NumPy AdamW oracle on {n} elements ({reps} steps), scaled by element count",
               "seconds_per_step": sec}
    out = {"metric": "AdamW step over the 8B-style model's embeddings, head and norms (HBM GB/s)",
           "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"AdamW leg: embedding and head {synth.ADAMW_VOCAB}x{synth.ADAMW_HIDDEN} bf16, "
                                  f"65 RMSNorm weights of {synth.ADAMW_HIDDEN}", "elements": elems,
                      "bytes_per_element": ADAMW_BYTES, "parallelism": "single GPU",
                      "hyperparameters": {"lr": ADAM_LR, "betas": list(ADAM_BETAS), "eps": ADAM_EPS,
                                          "weight_decay": ADAM_WD}},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS, "kernel": "adamw_kernel",
                        "traffic": measured_traffic("adamw_kernel_8b_nonmatrix_params.md", "adamw.hip", "bytes_per_step")},
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix
SOAP_LR, SOAP_WD, SOAP_MAX_DIM, SOAP_FREQ = 3e-4, 0.1, 8192, 10


def soap_flops(m, n, with_l, with_r, refresh=False):
    """Algorithmic flops of one SOAP update of an m x n matrix: the
    statistics (upper triangles), the rotations of G into the basis and of
    the direction back; with ``refresh`` the power-iteration product, the
    Householder QR (4/3 d^3 to factor, 4/3 d^3 to form Q) and the products
    that carry the first moment into the new basis, per side (two of m x n
    by d, or for one side alone on the shorter axis the d x d basis change
    and one of m x n by d)."""
    f = 0
    if with_l:
        f += m * (m + 1) * n + 2 * (2 * m * m * n)
        if refresh:
            # the moment's re-rotation: QL_new^T (QL_old mbar), or with the left
            # side alone and n > m, (QL_new^T QL_old) mbar
            carry = 2 * m ** 3 + 2 * m * m * n if (not with_r and n > m) else 2 * (2 * m * m * n)
            f += 2 * m ** 3 + (8 * m ** 3) // 3 + carry
    if with_r:
        f += n * (n + 1) * m + 2 * (2 * m * n * n)
        if refresh:
            carry = 2 * n ** 3 + 2 * m * n * n if (not with_l and m > n) else 2 * (2 * m * n * n)
            f += 2 * n ** 3 + (8 * n ** 3) // 3 + carry
    return f


def bench_soap(args):
    """Time SOAP steps (statistics, basis refresh every SOAP_FREQ steps,
    rotated Adam, update) over the layer's matrices; print one JSON line
    against the fp32 MFMA roofline."""
    import numpy as np
    import torch

    import matrix_aware_optimizer_step_amd as mx
    from matrix_aware_optimizer_step_amd import soap
    from workloads import synth

    mx._lib.load()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS[args.workload]
    grads = synth.group_gradients(cfg, step=1, device=dev)
    weights = synth.initial_weights(cfg, device=dev)
    step = soap.SoapStep(list(zip(weights, grads)), lr=SOAP_LR, weight_decay=SOAP_WD, freq=SOAP_FREQ,
                         max_dim=SOAP_MAX_DIM)
    torch.cuda.synchronize()
    log(f"[bench] SOAP over {cfg.slug}: {cfg.matrices} matrices, workspace {step.ws.numel() / 2**30:.2f} GiB")
    if args.copy_calibration:
        calibration_copy(dev)
    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    refreshes = 0
    t0 = time.perf_counter()
    for k in range(args.steps):
        refreshes += (step.t % step.freq) == 0      # the coming step refreshes
        step.step(events=events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps done in {wall:.3f} s ({refreshes} refreshes)")
    ph = [sum(e[i].elapsed_time(e[i + 1]) for e in events) / args.steps for i in range(4)]
    sides = [(g.count, g.rows, g.cols, g.rows <= SOAP_MAX_DIM, g.cols <= SOAP_MAX_DIM) for g in cfg.groups]
    base = sum(c * soap_flops(m, n, wl, wr) for c, m, n, wl, wr in sides)
    extra = sum(c * (soap_flops(m, n, wl, wr, True) - soap_flops(m, n, wl, wr)) for c, m, n, wl, wr in sides)
    flops = base + extra * refreshes / args.steps
    ms_per_step = wall * 1e3 / args.steps
    # the products outside the refresh: statistics and the rotations (the
    # precondition phase also runs the elementwise rotated-Adam kernel)
    gemm_ms = ph[0] + ph[2]
    gemm_tflops = base / (gemm_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import soap as OS
        g0 = next(g for g in cfg.groups if g.name == "wk_wv")
        G = grads[[g.name for g in cfg.groups].index("wk_wv")][0].double().cpu().numpy()
        W = np.zeros((g0.rows, g0.cols))
        st = OS.init_state(g0.rows, g0.cols, SOAP_MAX_DIM)
        t1 = time.perf_counter()
        OS.soap_step(W, G, st, lr=SOAP_LR, weight_decay=SOAP_WD, freq=SOAP_FREQ)
        t_ref = time.perf_counter() - t1
        t1 = time.perf_counter()
        OS.soap_step(W, G, st, lr=SOAP_LR, weight_decay=SOAP_WD, freq=SOAP_FREQ)
        t_plain = time.perf_counter() - t1
        fs_plain = soap_flops(g0.rows, g0.cols, True, True)
        fs_ref = soap_flops(g0.rows, g0.cols, True, True, True)
        rate_plain, rate_ref = fs_plain / t_plain, (fs_ref - fs_plain) / max(t_ref - t_plain, 1e-9)
        sec = base / rate_plain + extra / SOAP_FREQ / rate_ref
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            threads = os.cpu_count() or 1
        cpu = {"value": 1.0 / sec, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
               "sample": f"fp64 NumPy SOAP oracle: one {g0.rows}x{g0.cols} matrix, a step with refresh "
                         f"({t_ref:.1f} s) and one without ({t_plain:.1f} s); scaled by flops to the workload "
                         f"with one refresh per {SOAP_FREQ} steps",
               "seconds_per_step": sec}
    out = {"metric": "SOAP steps/sec + fp32 MFMA TFLOP/s of its products per layer set",
           "value": 1e3 / ms_per_step, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{cfg.slug} (SOAP): {cfg.name}", "matrices": cfg.matrices,
                      "shapes": {g.name: [g.count, g.rows, g.cols] for g in cfg.groups},
                      "preconditioned_sides": {g.name: [g.rows <= SOAP_MAX_DIM, g.cols <= SOAP_MAX_DIM]
                                               for g in cfg.groups},
                      "refresh_every": SOAP_FREQ, "refreshes_timed": refreshes,
                      "hyperparameters": {"lr": SOAP_LR, "weight_decay": SOAP_WD, "betas": [step.beta1, step.beta2],
                                          "eps": step.eps, "beta_s": step.beta_s, "max_dim": SOAP_MAX_DIM},
                      "parallelism": "single GPU"},
           "phases_ms": {"statistics": ph[0], "refresh": ph[1], "precondition": ph[2], "apply": ph[3]},
           "soap": {"flops_per_step": flops, "tflops": flops / (ms_per_step * 1e-3) / 1e12,
                    "flops_statistics_and_rotations": base, "flops_refresh": extra},
           "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": gemm_tflops / PEAK_FP32_MFMA_TFLOPS,
                        "traffic": measured_traffic("soap_sgemm_8b-dense-layer_hbm_traffic.md", "soap.hip",
                                                    "soap_products_bytes_per_step")
                        if cfg.slug == "8b-dense-layer" else None,
                        "kernel": "sgemm_list_kernel and sgemm_kernel (statistics and rotation products; timed "
                                  "with the rotated-Adam kernel of the precondition phase)"},
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, grads_host, budget_s=20.0, coeffs=COEFFS["quintic"][0], steps=5):
    """Time the fp64 oracle on a bounded sample of the workload's matrices
    (smallest first until about `budget_s` of work), scaled by NS flops to
    the whole workload."""
    import numpy as np
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    total_flops = sum(ns_flops(g.count, g.rows, g.cols, steps)[0] for g in cfg.groups)
    order = sorted(range(len(cfg.groups)), key=lambda i: cfg.groups[i].rows * cfg.groups[i].cols)
    spent, done_flops, names = 0.0, 0, []
    for gi in order:
        g = cfg.groups[gi]
        G = grads_host[gi].astype(np.float64)
        W = np.zeros((g.rows, g.cols))
        M = np.zeros((g.rows, g.cols))
        t0 = time.perf_counter()
        O.muon_step(W, M, G, lr=LR, weight_decay=WD, coeffs=coeffs, steps=steps)
        dt = time.perf_counter() - t0
        spent += dt
        done_flops += ns_flops(1, g.rows, g.cols, steps)[0]
        names.append(f"{g.name} {g.rows}x{g.cols}")
        if spent > budget_s * 0.5:
            break
    sec_per_step = spent * total_flops / done_flops
    return {"value": 1.0 / sec_per_step, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 NumPy oracle muon_step on one matrix each of [{', '.join(names)}] "
                      f"({spent:.1f} s), scaled by Newton-Schulz flops to the whole workload "
                      f"({cfg.matrices} matrices): extrapolated x{total_flops / done_flops:.1f}",
            "extrapolated": True, "scale_factor": total_flops / done_flops,
            "blas_threads": int(threads), "host_cpu_count": os.cpu_count(),
            "seconds_per_step": sec_per_step}


def main():
    from workloads.synth import BENCH_WORKLOADS

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8b-dense-32-layers", choices=BENCH_WORKLOADS)
    ap.add_argument("--coeffs", default="quintic", choices=sorted(COEFFS),
                    help="Newton-Schulz coefficient set (quintic: the Muon default)")
    ap.add_argument("--ns-steps", type=int, default=None, help="Newton-Schulz steps (default: the set's usual count)")
    ap.add_argument("--part", default="muon", choices=["muon", "adamw", "soap"],
                    help="muon: the Muon step of --workload (default); adamw: the AdamW step over the 8B-style "
                         "model's embeddings, head and norms; soap: SOAP steps over --workload's matrices")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-apply", action="store_true",
                    help="apply the update with its own kernel (muon_apply_grouped) instead of in the last "
                         "Newton-Schulz step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy before the warmup, so that profiler byte counters "
                         "can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the Muon step here runs on a single MI355X with no "
              f"collectives (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.part == "adamw":
        bench_adamw(args)
        return
    if args.part == "soap":
        bench_soap(args)
        return

    import numpy as np
    import torch

    import matrix_aware_optimizer_step_amd as mx
    from workloads import synth

    mx._lib.load()  # fails loudly without the HIP library
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS[args.workload]
    log(f"[bench] {cfg.slug}: {cfg.name}, {cfg.matrices} matrices, {cfg.elements / 1e6:.1f} M elements")

    t0 = time.perf_counter()
    grads = synth.group_gradients(cfg, step=1, device=dev)
    weights = synth.initial_weights(cfg, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    stepper = make_stepper(mx, weights, grads, args.coeffs, args.ns_steps, fused_apply=not args.separate_apply)
    fused = stepper.fused_apply
    ns_steps = stepper.steps
    if args.copy_calibration:
        calibration_copy(dev)

    def one_step(ev=None):
        stepper.step(events=ev)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    # exactly K steps, enqueued back to back; events on the same stream cut
    # them into up to five blocks of nearly equal step counts
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    nblocks = max(1, min(5, args.steps))
    sizes = [args.steps // nblocks + (1 if b < args.steps % nblocks else 0) for b in range(nblocks)]
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(nblocks + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bev[0].record()
    k = 0
    for b, size in enumerate(sizes):
        for _ in range(size):
            one_step(events[k])
            k += 1
        bev[b + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps done in {wall:.3f} s")
    block_rates = [sizes[b] / (bev[b].elapsed_time(bev[b + 1]) * 1e-3) for b in range(nblocks)]

    t_mom = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ns_times = sorted(e[1].elapsed_time(e[2]) for e in events)
    t_ns = sum(ns_times) / args.steps
    t_app = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    algo, nominal = 0, 0
    for g in cfg.groups:
        fa, fn = ns_flops(g.count, g.rows, g.cols, ns_steps)
        algo += fa
        nominal += fn
    ns_tflops = algo / (t_ns * 1e-3) / 1e12
    ns_tflops_nominal = nominal / (t_ns * 1e-3) / 1e12
    elems = cfg.elements
    mom_bytes = momentum_bytes(cfg, stepper.packed)
    app_bytes = elems * (4 + 2)       # W bf16 read+write, O bf16 read
    mom_gbs = mom_bytes / (t_mom * 1e-3) / 1e9
    app_gbs = None if fused else app_bytes / (t_app * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a bounded sample (host cores)")
        host = [g[0].float().cpu().numpy() for g in grads]
        cpu = cpu_baseline(cfg, host, coeffs=stepper.coeffs, steps=ns_steps)
        log(f"[bench] oracle: {cpu['seconds_per_step']:.1f} s per step (extrapolated)")

    shapes = {g.name: [g.count, g.rows, g.cols] for g in cfg.groups}
    out = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.slug}: {cfg.name}", "matrices": cfg.matrices,
                   "shapes": shapes, "gradients": cfg.kind, "ns_steps": ns_steps, "coefficients": args.coeffs,
                   "compute": "bf16 MFMA, fp32 accumulate",
                   "hyperparameters": {"beta": stepper.beta, "nesterov": bool(stepper.nesterov), "eps": stepper.eps,
                                       "abc": [float(x) for x in stepper.coeffs], "lr": stepper.lr,
                                       "weight_decay": stepper.weight_decay,
                                       "scale": f"{stepper.coeff}*sqrt(max(m,n))", "momentum_dtype": "f32",
                                       "ns_input_dtype": ("bf16 high part + 8-bit residual, written by the momentum "
                                                          "kernel" if stepper.packed else "f32")},
                   "parallelism": "single GPU"},
        "repeats": {"blocks": nblocks, "steps_per_block": sizes, "steps_per_s": block_rates,
                    "median_steps_per_s": float(np.median(block_rates)), "min_steps_per_s": min(block_rates),
                    "max_steps_per_s": max(block_rates)},
        "newton_schulz": {"tflops_algorithmic": ns_tflops, "tflops_nominal_4m2n_2m3": ns_tflops_nominal,
                          "frac_bf16_peak": ns_tflops / PEAK_BF16_TFLOPS, "ms": t_ns,
                          "ms_median": float(np.median(ns_times)), "ms_min": ns_times[0], "ms_max": ns_times[-1],
                          "tflops_algorithmic_median": algo / (float(np.median(ns_times)) * 1e-3) / 1e12,
                          "flops_algorithmic": algo, "flops_nominal": nominal},
        "elementwise": {"momentum_ms": t_mom, "momentum_gbs": mom_gbs, "momentum_frac_hbm": mom_gbs / PEAK_HBM_GBS,
                        "apply_ms": None if fused else t_app, "apply_gbs": app_gbs,
                        "apply_frac_hbm": None if fused else app_gbs / PEAK_HBM_GBS,
                        "apply": ("in the last Newton-Schulz step's epilogue (reads and writes W, O never stored; "
                                  "its time is in newton_schulz.ms)" if fused else "muon_apply_grouped")},
        "roofline": {"bound": "mfma", "achieved": ns_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ns_tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(f"ns_gemm_{cfg.slug}_hbm_traffic.md", "ns_gemm.hip",
                                                                    "ns_gemm_bytes_per_step"),
                     "kernel": ("ns_gemm_kernel (Gram, polynomial and update launches of "
                                f"{ns_call(stepper)}"
                                "; achieved over the whole call, traffic over the ns_gemm_kernel launches)")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
