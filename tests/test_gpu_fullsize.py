"""Parity at the workloads' full sizes, in the benchmark's launch configuration.

Each test builds one whole workload at its real shapes on the GPU, runs one
optimizer step through ``bench.make_stepper`` (the very grouped launches the
benchmark times) and compares a sample of the matrices with the fp64 oracle
run on the same seeded inputs:

* momentum (fp32) and sum of squares: relative error <= 1e-6;
* Newton-Schulz output (bf16 MFMA path): relative Frobenius error <= 3e-2;
* the updated bf16 weight: within one bf16 rounding of the oracle's apply
  step evaluated on the GPU's own Newton-Schulz output.

Sampled matrices get their workload's gradient recipe; the others get a
seeded Gaussian of the same shape, which keeps the launch identical while
sparing the host the cost of generating what is not checked.  Sampled
indices include the last matrix of large groups, so per-matrix offsets far
from the base are exercised.
"""

import time

import numpy as np
import pytest
import torch

import bench
from oracle import oracle as O
from workloads import synth

pytestmark = pytest.mark.gpu

TOL_EW = 1e-6
TOL_BF16 = 3e-2

# workload -> {group name: matrix indices within the group to check}
SAMPLES = {
    "8b-dense-layer": {"wq_wo": [0], "wk_wv": [1], "gate_up": [1], "down": [0]},
    "8b-dense-32-layers": {"wq_wo": [63], "wk_wv": [0], "gate_up": [37], "down": [31]},
    "moe-30b-a3b-layer": {"gate_up": list(range(0, 256, 16)) + [255], "down": list(range(3, 128, 16)) + [127]},
    "qkv-heads-kappa1e4": {"qkv_heads": list(range(96)), "gate_up": [1], "down": [0]},
}


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()  # raises when the library is missing: there is no fallback
    return m


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_of(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def gradients(cfg, dev, picks):
    """Per group a (count, rows, cols) tensor: the recipe for picked matrices,
    a seeded Gaussian filler elsewhere."""
    counts = synth.moe_token_counts(synth.seed_of(cfg.seed_id, 0, 0), device=dev) if cfg.kind == "moe" else None
    out, i = [], 0
    for grp in cfg.groups:
        t = torch.empty(grp.count, grp.rows, grp.cols, dtype=cfg.dtype, device=dev)
        for k in range(grp.count):
            if k in picks.get(grp.name, ()):
                t[k] = synth.gradient(cfg, i, grp.rows, grp.cols, 1, dev, counts).to(cfg.dtype)
            else:
                t[k] = synth.gaussian(grp.rows, grp.cols, synth.seed_of(cfg.seed_id, i, 1), dev).to(cfg.dtype)
            i += 1
        out.append(t)
    return out


@pytest.mark.parametrize("workload", list(synth.BENCH_WORKLOADS))
def test_full_size_step_matches_oracle(mx, workload):
    cfg = synth.WORKLOADS[workload]
    picks = SAMPLES[workload]
    dev = torch.device("cuda:0")
    print(f"[fullsize] {workload}: {cfg.name}", flush=True)
    grads = gradients(cfg, dev, picks)
    weights = synth.initial_weights(cfg, device=dev)
    w0 = {(gi, k): f64(weights[gi][k]) for gi, grp in enumerate(cfg.groups) for k in picks.get(grp.name, ())}
    stepper = bench.make_stepper(mx, weights, grads)
    stepper.step()
    torch.cuda.synchronize()
    print(f"[fullsize] {workload}: GPU step done", flush=True)

    worst = {"mom": 0.0, "sumsq": 0.0, "ortho": 0.0}
    ortho_errs = []
    t0 = time.perf_counter()
    for gi, grp in enumerate(cfg.groups):
        for k in picks.get(grp.name, ()):
            G = f64(grads[gi][k])
            W_new, M_new, O_want, ss_want = O.muon_step(w0[(gi, k)], np.zeros_like(G), G,
                                                        lr=stepper.lr, weight_decay=stepper.weight_decay)
            e_mom = O.relative_frobenius_error(f64(stepper.momentum_buffers[gi][k]), M_new)
            e_ss = abs(float(stepper.sumsq_buffers[gi][k]) - ss_want) / ss_want
            O_got = f64(stepper.ortho_buffers[gi][k])
            e_o = O.relative_frobenius_error(O_got, O_want)
            ortho_errs.append(e_o)
            where = f"{workload} {grp.name}[{k}] {grp.rows}x{grp.cols}"
            assert e_mom <= TOL_EW, f"{where}: momentum error {e_mom:.3g}"
            assert e_ss <= TOL_EW, f"{where}: sum of squares error {e_ss:.3g}"
            assert e_o <= TOL_BF16, f"{where}: Newton-Schulz error {e_o:.3g}"
            # the apply kernel on the GPU's own O against the oracle's apply step
            W_exact = O.apply_update(w0[(gi, k)], O_got, stepper.lr, stepper.weight_decay)
            W_got = f64(weights[gi][k])
            tol = bf16_ulp(W_exact) + TOL_EW * np.max(np.abs(W_exact))
            assert np.all(np.abs(W_got - bf16_of(W_exact)) <= tol), f"{where}: updated weight"
            worst = {"mom": max(worst["mom"], e_mom), "sumsq": max(worst["sumsq"], e_ss),
                     "ortho": max(worst["ortho"], e_o)}
    print(f"[fullsize] {workload}: oracle checks {time.perf_counter() - t0:.1f} s, worst errors "
          f"momentum {worst['mom']:.2e} sumsq {worst['sumsq']:.2e} Newton-Schulz {worst['ortho']:.2e} "
          f"(median over {len(ortho_errs)} sampled matrices {float(np.median(ortho_errs)):.2e})", flush=True)
    del stepper, grads, weights
    torch.cuda.empty_cache()
