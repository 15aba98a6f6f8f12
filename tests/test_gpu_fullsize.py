"""Parity at the workloads' full sizes, in the benchmark's launch configuration.

Each test builds one whole workload at its real shapes on the GPU, runs one
optimizer step through ``bench.make_stepper`` (the very grouped launches the
benchmark times) and compares a sample of the matrices with the fp64 oracle
run on the same seeded inputs:

* momentum (fp32) and sum of squares: relative error <= 1e-6;
* Newton-Schulz output (bf16 MFMA path): relative Frobenius error <= 3e-2;
* the updated bf16 weight: within one bf16 rounding of the oracle's apply
  step evaluated on the GPU's own Newton-Schulz output.

The benchmark applies the update in the last Newton-Schulz step, so its O
is never stored.  Each test therefore runs that step first and keeps the
sampled weights, puts the sampled matrices back to their starting values and
runs a second step with the separate apply call, whose O and W are checked
against the oracle as above; the first step's weights must lie within one
bf16 unit plus lr*s*2^-8 |O| of the second's (the rounding of O to bf16 that
only the separate call takes).

Sampled matrices get their workload's gradient recipe; the others get a
seeded Gaussian of the same shape, which keeps the launch identical while
sparing the host the cost of generating what is not checked.  Sampled
indices include the last matrix of large groups, so per-matrix offsets far
from the base are exercised.

The 32-layer set is checked on every matrix of three whole layers: the
first, the last and one drawn from a fixed seed (21 matrices).  Its GPU step
runs once per module; each layer is then one test, so that the fp64 oracle's
work (about a minute per layer on the host) stays within one test's time.
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
# the 32-layer set: layers 0 and 31 and one seeded layer, all 7 matrices of each
# (layer L holds wq_wo 2L, 2L+1; wk_wv 2L, 2L+1; gate_up 2L, 2L+1; down L)
LAYERS_32 = (0, int(np.random.default_rng(3_000_000).integers(1, 31)), 31)


def layer_picks(layers):
    return {"wq_wo": [i for L in layers for i in (2 * L, 2 * L + 1)],
            "wk_wv": [i for L in layers for i in (2 * L, 2 * L + 1)],
            "gate_up": [i for L in layers for i in (2 * L, 2 * L + 1)],
            "down": list(layers)}


SAMPLES = {
    "8b-dense-layer": {"wq_wo": [0], "wk_wv": [1], "gate_up": [1], "down": [0]},
    "8b-dense-32-layers": layer_picks(LAYERS_32),
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


def two_steps(mx, cfg, weights, grads, picks):
    """The benchmark's step (update in the last Newton-Schulz step), then the
    separate-apply step on the same inputs for the sampled matrices.  Returns
    the second stepper and {(group index, k): weight after the first step}."""
    w0 = {(gi, k): weights[gi][k].clone() for gi, grp in enumerate(cfg.groups) for k in picks.get(grp.name, ())}
    fused = bench.make_stepper(mx, weights, grads)
    assert fused.fused_apply
    fused.step()
    torch.cuda.synchronize()
    w_fused = {key: weights[key[0]][key[1]].cpu() for key in w0}
    del fused
    for (gi, k), w in w0.items():
        weights[gi][k].copy_(w)
    sep = bench.make_stepper(mx, weights, grads, fused_apply=False)
    sep.step()
    torch.cuda.synchronize()
    return sep, w_fused


def check_fused(w_fused, w_sep, o_sep, lr, rows, cols, where):
    step = lr * O.scale_factor(rows, cols, O.SCALE_MATCH_RMS, 0.2)
    tol = bf16_ulp(np.maximum(np.abs(w_fused), np.abs(w_sep))) + step * 2.0 ** -8 * np.abs(o_sep)
    bad = int((np.abs(w_fused - w_sep) > tol).sum())
    assert bad == 0, f"{where}: {bad} elements of the fused update beyond one rounding of the separate apply"


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


@pytest.mark.parametrize("workload", [w for w in synth.BENCH_WORKLOADS if w != "8b-dense-32-layers"])
def test_full_size_step_matches_oracle(mx, workload):
    cfg = synth.WORKLOADS[workload]
    picks = SAMPLES[workload]
    dev = torch.device("cuda:0")
    print(f"[fullsize] {workload}: {cfg.name}", flush=True)
    grads = gradients(cfg, dev, picks)
    weights = synth.initial_weights(cfg, device=dev)
    w0 = {(gi, k): f64(weights[gi][k]) for gi, grp in enumerate(cfg.groups) for k in picks.get(grp.name, ())}
    stepper, w_fused = two_steps(mx, cfg, weights, grads, picks)
    print(f"[fullsize] {workload}: GPU steps done", flush=True)

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
            check_fused(f64(w_fused[(gi, k)]), W_got, O_got, stepper.lr, grp.rows, grp.cols, where)
            worst = {"mom": max(worst["mom"], e_mom), "sumsq": max(worst["sumsq"], e_ss),
                     "ortho": max(worst["ortho"], e_o)}
    print(f"[fullsize] {workload}: oracle checks {time.perf_counter() - t0:.1f} s, worst errors "
          f"momentum {worst['mom']:.2e} sumsq {worst['sumsq']:.2e} Newton-Schulz {worst['ortho']:.2e} "
          f"(median over {len(ortho_errs)} sampled matrices {float(np.median(ortho_errs)):.2e})", flush=True)
    del stepper, grads, weights
    torch.cuda.empty_cache()


# ------------------------------------------------------ the 32-layer set

ERRS_32 = []


@pytest.fixture(scope="module")
def step_32(mx):
    """One optimizer step of the whole 32-layer set through the benchmark's
    launches; host copies of the sampled matrices' inputs and outputs."""
    workload = "8b-dense-32-layers"
    cfg = synth.WORKLOADS[workload]
    picks = SAMPLES[workload]
    dev = torch.device("cuda:0")
    print(f"[fullsize] {workload}: layers {LAYERS_32}, generating inputs", flush=True)
    grads = gradients(cfg, dev, picks)
    weights = synth.initial_weights(cfg, device=dev)
    host = {}
    for gi, grp in enumerate(cfg.groups):
        for k in picks[grp.name]:
            host[(grp.name, k)] = {"G": grads[gi][k].cpu(), "W0": weights[gi][k].cpu()}
    stepper, w_fused = two_steps(mx, cfg, weights, grads, picks)
    print(f"[fullsize] {workload}: GPU steps done", flush=True)
    for gi, grp in enumerate(cfg.groups):
        for k in picks[grp.name]:
            host[(grp.name, k)].update(M=stepper.momentum_buffers[gi][k].cpu(), O=stepper.ortho_buffers[gi][k].cpu(),
                                      W=weights[gi][k].cpu(), W_fused=w_fused[(gi, k)],
                                      sumsq=float(stepper.sumsq_buffers[gi][k]))
    lr, wd = stepper.lr, stepper.weight_decay
    del stepper, grads, weights
    torch.cuda.empty_cache()
    return host, lr, wd


@pytest.mark.parametrize("layer", LAYERS_32)
def test_32_layer_set_sampled_layer_matches_oracle(step_32, layer):
    host, lr, wd = step_32
    picks = layer_picks([layer])
    t0 = time.perf_counter()
    for name, ks in picks.items():
        for k in ks:
            h = host[(name, k)]
            G, W0 = f64(h["G"]), f64(h["W0"])
            W_new, M_new, O_want, ss_want = O.muon_step(W0, np.zeros_like(G), G, lr=lr, weight_decay=wd)
            where = f"8b-dense-32-layers layer {layer} {name}[{k}] {G.shape[0]}x{G.shape[1]}"
            e_mom = O.relative_frobenius_error(f64(h["M"]), M_new)
            e_ss = abs(h["sumsq"] - ss_want) / ss_want
            O_got = f64(h["O"])
            e_o = O.relative_frobenius_error(O_got, O_want)
            ERRS_32.append(e_o)
            print(f"[fullsize] {where}: Newton-Schulz {e_o:.3e} momentum {e_mom:.1e} sumsq {e_ss:.1e}", flush=True)
            assert e_mom <= TOL_EW, f"{where}: momentum error {e_mom:.3g}"
            assert e_ss <= TOL_EW, f"{where}: sum of squares error {e_ss:.3g}"
            assert e_o <= TOL_BF16, f"{where}: Newton-Schulz error {e_o:.3g}"
            W_exact = O.apply_update(W0, O_got, lr, wd)
            tol = bf16_ulp(W_exact) + TOL_EW * np.max(np.abs(W_exact))
            assert np.all(np.abs(f64(h["W"]) - bf16_of(W_exact)) <= tol), f"{where}: updated weight"
            check_fused(f64(h["W_fused"]), f64(h["W"]), O_got, lr, G.shape[0], G.shape[1], where)
    print(f"[fullsize] 8b-dense-32-layers layer {layer}: oracle {time.perf_counter() - t0:.1f} s; over the "
          f"{len(ERRS_32)} matrices checked so far Newton-Schulz worst {max(ERRS_32):.3e} "
          f"median {float(np.median(ERRS_32)):.3e}", flush=True)
