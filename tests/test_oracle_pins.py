"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Nothing here re-types the oracle's formulas.  Each test checks the oracle
against a different route to the same number:

* values the pages print (golden JSON files under tests/golden/, each with
  its citation);
* Lemma 3 of "Matrix optimizers: K-FAC, Shampoo and Muon" (the step acts on
  singular values only), evaluated through an SVD and a scalar map;
* the exact polar factor from an SVD, and from Shampoo's inverse fourth
  roots (Proposition 4 of the same lesson) via scipy;
* closed forms of the moving average and of repeated decoupled decay
  ("LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
  Training", sections 5 and 6);
* invariants: transpose equivariance, scale invariance, odd symmetry.

The last test plants plausible mistakes in the oracle (on the CPU) and
checks that at least one pin catches each of them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.linalg import fractional_matrix_power

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def svd_polar(G):
    U, s, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    return U @ Vt


def scalar_map(sigma, coeffs, steps):
    a, b, c = coeffs
    x = np.array(sigma, dtype=np.float64)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def lemma3_closed_form(N, coeffs, steps, eps):
    """U p^{K}(S / (||N||_F + eps)) V^T from an SVD (Lemma 3)."""
    N = np.asarray(N, dtype=np.float64)
    U, s, Vt = np.linalg.svd(N, full_matrices=False)
    s0 = s / (np.linalg.norm(s) + eps)
    return (U * scalar_map(s0, coeffs, steps)) @ Vt


def haar(rng, n, k):
    """n x k matrix with orthonormal columns (sign-fixed QR of a Gaussian)."""
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def with_spectrum(rng, m, n, sigma):
    r = len(sigma)
    return (haar(rng, m, r) * np.asarray(sigma)) @ haar(rng, n, r).T


# ---------------------------------------------------------------- worked 2x2

def test_worked_example_fixture_is_consistent():
    g = golden("worked_example_2x2.json")
    G = np.array(g["G"])
    s = np.linalg.svd(G, compute_uv=False)
    np.testing.assert_allclose(s.round(4), g["singular_values_4dp"])
    np.testing.assert_allclose(math.sqrt(5) * svd_polar(G), g["polar_times_sqrt5"], atol=1e-12)
    np.testing.assert_allclose((s / np.linalg.norm(G)).round(3), g["normalized_singular_values_3dp"])


def _per_direction(G, X):
    U, _, Vt = np.linalg.svd(G)
    return np.array([U[:, i] @ X @ Vt[i] for i in range(2)]), U, Vt


def test_worked_example_quintic_trajectory_per_direction():
    g = golden("worked_example_2x2.json")
    G = np.array(g["G"])
    for k, want in enumerate(g["quintic_per_direction_3dp"], start=1):
        X = O.newton_schulz(G, k, O.QUINTIC)
        got, U, Vt = _per_direction(G, X)
        np.testing.assert_allclose(got.round(3), want, atol=1e-12, err_msg=f"step {k}")
        # singular vectors are kept: no cross terms (Lemma 3)
        assert abs(U[:, 0] @ X @ Vt[1]) < 1e-12 and abs(U[:, 1] @ X @ Vt[0]) < 1e-12


def test_worked_example_quintic_ns5_singular_values():
    g = golden("worked_example_2x2.json")
    X = O.newton_schulz(np.array(g["G"]), 5, O.QUINTIC)
    np.testing.assert_allclose(np.linalg.svd(X, compute_uv=False).round(3),
                               g["quintic_ns5_singular_values_3dp"])


def test_worked_example_cubic_trajectory_and_convergence():
    g = golden("worked_example_2x2.json")
    G = np.array(g["G"])
    for k, want in enumerate(g["cubic_per_direction_3dp"], start=1):
        got, _, _ = _per_direction(G, O.newton_schulz(G, k, O.CUBIC))
        np.testing.assert_allclose(got.round(3), want, atol=1e-12, err_msg=f"step {k}")
    Q = svd_polar(G)
    e6 = np.abs(O.newton_schulz(G, 6, O.CUBIC) - Q).max()
    e7 = np.abs(O.newton_schulz(G, 7, O.CUBIC) - Q).max()
    assert 1e-6 < e6 < 5e-5          # printed: about 1e-5 after 6 steps
    assert e7 < 1e-9                 # printed: about 1e-10 after 7 steps


def test_theorem2_inner_products_and_converged_oracle():
    g = golden("worked_example_2x2.json")
    G = np.array(g["G"])
    s = np.linalg.svd(G, compute_uv=False)
    sg = np.sign(G)
    want = g["inner_product_4dp"]
    assert round(float(np.sum(G * svd_polar(G))), 4) == want["polar"]
    assert round(float(np.sum(G * G / s[0])), 4) == want["G_over_sigma1"]
    assert round(float(np.sum(G * sg / np.linalg.norm(sg, 2))), 4) == want["sign_normalized"]
    assert round(float(s.sum()), 4) == g["nuclear_norm_4dp"]
    # the converged oracle attains the nuclear norm (Theorem 2)
    X = O.newton_schulz(G, 30, O.CUBIC)
    assert abs(np.sum(G * X) - s.sum()) < 1e-9


def test_shampoo_route_matches_converged_oracle():
    g = golden("worked_example_2x2.json")
    rng = np.random.default_rng(3)
    for G in (np.array(g["G"]), rng.standard_normal((8, 5)), rng.standard_normal((5, 9))):
        conv = O.newton_schulz(G, 60, O.CUBIC)
        for k, f in zip(g["shampoo_identical_gradients"]["k"], g["shampoo_identical_gradients"]["factor"]):
            S = (fractional_matrix_power(k * G @ G.T, -0.25) @ G
                 @ fractional_matrix_power(k * G.T @ G, -0.25))
            if G.shape[0] != G.shape[1]:
                continue  # the inverse roots of the rank-deficient Gram need the range projector
            np.testing.assert_allclose(np.real(S), f * conv, atol=1e-9)
        # rectangular: compare on the range via the SVD polar factor
        np.testing.assert_allclose(conv, svd_polar(G), atol=1e-9)


# ---------------------------------------------------------- quintic scalar map

def test_quintic_p_of_one_and_rank_one_input():
    q = golden("quintic_scalar_map.json")
    assert tuple(q["coefficients"]) == O.QUINTIC
    rng = np.random.default_rng(0)
    G = np.outer(rng.standard_normal(6), rng.standard_normal(9))
    unit = G / np.linalg.norm(G)
    X1 = O.newton_schulz(G, 1, O.QUINTIC)
    ratio = np.sum(X1 * unit)
    assert round(float(ratio), 3) == q["p_of_one_3dp"]
    np.testing.assert_allclose(X1, ratio * unit, atol=1e-12)
    X5 = O.newton_schulz(G, 5, O.QUINTIC)
    np.testing.assert_allclose(X5, scalar_map(1.0, O.QUINTIC, 5) * unit, atol=1e-6)


def test_quintic_trajectory_from_0p01():
    q = golden("quintic_scalar_map.json")
    rng = np.random.default_rng(1)
    big, small = q["two_direction_example"]["normalized"]
    sig = [math.sqrt(1.0 - small ** 2), small, 0.0]
    U, V = haar(rng, 3, 3), haar(rng, 7, 3)
    N = (U * sig) @ V.T
    traj = []
    for k in range(1, 6):
        X = O.newton_schulz(N, k, O.QUINTIC)
        traj.append(U[:, 1] @ X @ V[:, 1])
    np.testing.assert_allclose(np.round(traj, 3), q["trajectory_from_0p01_3dp"])
    X = O.newton_schulz(N, 5, O.QUINTIC)
    got = [U[:, 0] @ X @ V[:, 0], U[:, 1] @ X @ V[:, 1]]
    np.testing.assert_allclose(np.round(got, 3), q["two_direction_example"]["after_5_steps_3dp"])
    assert abs(U[:, 2] @ X @ V[:, 2]) < 1e-14  # p(0) = 0


def test_quintic_band_after_five_steps():
    q = golden("quintic_scalar_map.json")
    lo, hi = q["band_after_5_steps"]["output_range_2dp"]
    rng = np.random.default_rng(2)
    seen = []
    for t in np.geomspace(0.01, 0.7, 25):
        N = with_spectrum(rng, 4, 6, [math.sqrt(1 - t * t), t])
        s = np.linalg.svd(O.newton_schulz(N, 5, O.QUINTIC), compute_uv=False)[:2]
        seen.extend(s)
    assert round(min(seen), 2) >= lo and round(max(seen), 2) <= hi
    assert round(min(seen), 2) == lo  # the band's ends are reached, not just respected


def test_example_64x256_band_and_update_rms():
    e = golden("example_64x256.json")
    rng = np.random.default_rng(0)
    sig = np.geomspace(e["singular_values"]["geomspace_from"], e["singular_values"]["geomspace_to"],
                       e["singular_values"]["count"])
    G2 = with_spectrum(rng, e["rows"], e["cols"], sig)
    O2 = O.newton_schulz(G2, 5, O.QUINTIC)
    sv = np.linalg.svd(O2, compute_uv=False)
    assert round(float(sv.min()), 2) == e["ns5_singular_value_min_2dp"]
    assert round(float(sv.max()), 2) == e["ns5_singular_value_max_2dp"]
    upd = O.apply_update(np.zeros_like(O2), O2, lr=1.0, weight_decay=0.0,
                         mode=O.SCALE_MATCH_RMS, coeff=0.2)
    assert round(float(np.sqrt(np.mean(upd ** 2))), 3) == e["update_rms_match_rms_3dp"]


# ------------------------------------------------------------ Lemma 3 / polar

@pytest.mark.parametrize("shape,rank", [((48, 80), None), ((80, 48), None), ((64, 64), None),
                                        ((40, 60), 10), ((1, 33), None), ((33, 1), None)])
@pytest.mark.parametrize("coeffs,steps", [(O.QUINTIC, 5), (O.CUBIC, 3), (O.TRACK3, 12), (O.QUINTIC, 0)])
def test_lemma3_closed_form(shape, rank, coeffs, steps):
    rng = np.random.default_rng(hash((shape, rank, steps)) % 2 ** 32)
    m, n = shape
    if rank is None:
        N = rng.standard_normal(shape) * 3.0
    else:
        N = rng.standard_normal((m, rank)) @ rng.standard_normal((rank, n))
    got = O.newton_schulz(N, steps, coeffs, O.EPS)
    want = lemma3_closed_form(N, coeffs, steps, O.EPS)
    assert O.relative_frobenius_error(got, want) < 1e-12


def test_converged_output_is_the_svd_polar_factor():
    rng = np.random.default_rng(10)
    N = rng.standard_normal((256, 128))
    Q = svd_polar(N)
    assert np.abs(O.newton_schulz(N, 12, O.TRACK3) - Q).max() < 1e-6
    assert np.abs(O.newton_schulz(N, 40, O.CUBIC) - Q).max() < 1e-10
    assert np.abs(O.newton_schulz(N.T, 40, O.CUBIC) - Q.T).max() < 1e-10


def test_orthogonal_input_direction_unchanged():
    rng = np.random.default_rng(11)
    for m, n in ((64, 64), (32, 128), (128, 32)):
        Q = haar(rng, max(m, n), min(m, n))
        Q = Q if m >= n else Q.T
        r = min(m, n)
        X = O.newton_schulz(Q, 5, O.QUINTIC)
        c = scalar_map(1.0 / (math.sqrt(r) + O.EPS), O.QUINTIC, 5)
        np.testing.assert_allclose(X, c * Q, atol=1e-12)
        # with the convergent cubic the input comes back unchanged
        np.testing.assert_allclose(O.newton_schulz(Q, 40, O.CUBIC), Q, atol=1e-12)


def test_transpose_equivariance():
    rng = np.random.default_rng(12)
    for shape in ((30, 70), (70, 30)):
        N = rng.standard_normal(shape)
        assert np.array_equal(O.newton_schulz(N.T, 5), O.newton_schulz(N, 5).T)
    S = rng.standard_normal((40, 40))
    np.testing.assert_allclose(O.newton_schulz(S.T, 5), O.newton_schulz(S, 5).T, atol=1e-13)


def test_scale_invariance_odd_symmetry_and_zero():
    rng = np.random.default_rng(13)
    N = rng.standard_normal((24, 56))
    base = O.newton_schulz(N, 5)
    assert O.relative_frobenius_error(O.newton_schulz(1000.0 * N, 5), base) < 1e-7
    assert np.array_equal(O.newton_schulz(-N, 5), -base)
    Z = O.newton_schulz(np.zeros((5, 7)), 5)
    assert np.all(Z == 0.0)


# --------------------------------------------------------------- momentum

def test_momentum_three_step_closed_form():
    rng = np.random.default_rng(20)
    beta = 0.95
    Gs = [rng.standard_normal((6, 9)) for _ in range(3)]
    M = np.zeros((6, 9))
    for G in Gs:
        M, N = O.momentum(M, G, beta, nesterov=False)
        np.testing.assert_array_equal(N, M)
    geo = (1 - beta) * (beta ** 2 * Gs[0] + beta * Gs[1] + Gs[2])
    np.testing.assert_allclose(M, geo, rtol=1e-14, atol=1e-15)


def test_momentum_constant_gradient_mass():
    # E[m_t] = (1 - beta^t) mu for a constant gradient ("LLM Optimizers", section 5)
    beta, G = 0.9, np.full((3, 3), 2.5)
    M = np.zeros((3, 3))
    for t in range(1, 8):
        M, _ = O.momentum(M, G, beta, nesterov=False)
        np.testing.assert_allclose(M, (1 - beta ** t) * G, rtol=1e-14)


def test_ema_and_accumulating_forms_give_the_same_update():
    rng = np.random.default_rng(21)
    beta = 0.95
    M = np.zeros((16, 40))
    B = np.zeros((16, 40))
    for _ in range(4):
        G = rng.standard_normal((16, 40))
        M, N = O.momentum(M, G, beta, nesterov=True)
        B = beta * B + G                         # accumulating form of the pages
        Nacc = G + beta * B
        np.testing.assert_allclose(N, (1 - beta) * Nacc, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(O.newton_schulz(N, 5), O.newton_schulz(Nacc, 5), rtol=0, atol=1e-6)


# ----------------------------------------------------------------- apply

def test_update_rms_of_exact_polar_factor():
    u = golden("update_rms.json")
    rng = np.random.default_rng(30)
    mm = u["mlp_3072x768"]
    m, n = mm["rows"], mm["cols"]
    Q = haar(rng, m, n)
    rms = lambda x: float(np.sqrt(np.mean(x ** 2)))
    assert round(rms(Q), 3) == mm["polar_rms_3dp"]
    W0 = np.zeros((m, n))
    orig = O.apply_update(W0, Q, 1.0, 0.0, O.SCALE_ORIGINAL)
    assert round(rms(orig), 3) == mm["original_rms_3dp"]
    assert round(O.scale_factor(m, n, O.SCALE_MATCH_RMS, 0.2), 1) == mm["match_rms_factor_1dp"]
    match = O.apply_update(W0, Q, 1.0, 0.0, O.SCALE_MATCH_RMS, 0.2)
    assert round(rms(match), 1) == mm["match_rms_rms_1dp"]
    assert abs(rms(match) - 0.2) < 1e-12
    qc = u["quick_check_1024x4096"]
    Q2 = haar(rng, qc["cols"], qc["rows"]).T
    lr = 3e-4
    upd = O.apply_update(np.zeros_like(Q2), Q2, lr, 0.0)
    assert abs(rms(upd) / lr - qc["update_rms_over_lr"]) < 1e-12
    # decoupled decay: the decay multiplies W only, so the update term keeps
    # its RMS whatever the weight decay is
    upd_wd = O.apply_update(np.zeros_like(Q2), Q2, lr, 0.5)
    assert abs(rms(upd_wd) / lr - qc["update_rms_over_lr"]) < 1e-12


def test_zero_gradient_gives_pure_decay_product():
    # theta_T = theta_0 * prod (1 - eta lambda) ("LLM Optimizers", section 6)
    rng = np.random.default_rng(31)
    W0 = rng.standard_normal((12, 20))
    W, M = W0.copy(), np.zeros_like(W0)
    lr, wd, T = 0.01, 0.5, 6
    for _ in range(T):
        W, M, Ot, sumsq = O.muon_step(W, M, np.zeros_like(W0), lr=lr, weight_decay=wd)
        assert sumsq == 0.0 and np.all(Ot == 0.0)
    np.testing.assert_allclose(W, (1 - lr * wd) ** T * W0, rtol=1e-13)


def test_scale_modes():
    assert O.scale_factor(3072, 768, O.SCALE_ORIGINAL) == 2.0
    assert O.scale_factor(768, 3072, O.SCALE_ORIGINAL) == 1.0
    assert O.scale_factor(5, 7, O.SCALE_NONE) == 1.0
    beta = 0.95
    kimi = math.sqrt((1 - beta) / (1 + beta))
    assert abs(kimi - 0.160) < 1e-3
    assert abs(O.scale_factor(100, 400, O.SCALE_MATCH_RMS, kimi) - kimi * 20) < 1e-12


def test_invalid_arguments():
    with pytest.raises(ValueError):
        O.momentum(np.zeros((2, 2)), np.zeros((2, 3)))
    with pytest.raises(ValueError):
        O.momentum(np.zeros((2, 2)), np.zeros((2, 2)), beta=1.0)
    with pytest.raises(ValueError):
        O.newton_schulz(np.zeros((2, 2)), -1)
    with pytest.raises(ValueError):
        O.scale_factor(2, 2, 7)


def test_apply_superposition():
    """The update is affine with a decay term in W and a separate term in O:
    apply(W, O) = apply(W, 0) + apply(0, O).  Together with the decay
    product and the update-RMS pins this fixes the combined formula."""
    rng = np.random.default_rng(32)
    W, Ot = rng.standard_normal((20, 12)), rng.standard_normal((20, 12))
    for mode in (O.SCALE_MATCH_RMS, O.SCALE_ORIGINAL, O.SCALE_NONE):
        both = O.apply_update(W, Ot, 0.7, 0.3, mode)
        parts = O.apply_update(W, np.zeros_like(Ot), 0.7, 0.3, mode) + O.apply_update(np.zeros_like(W), Ot, 0.7, 0.3, mode)
        np.testing.assert_allclose(both, parts, rtol=1e-14, atol=1e-14)


# ------------------------------------------------- planted mistakes are caught

def _run_pins():
    """Run the value pins; return the names of those that fail."""
    fails = []
    for fn in (test_worked_example_quintic_trajectory_per_direction,
               test_worked_example_cubic_trajectory_and_convergence,
               test_quintic_p_of_one_and_rank_one_input,
               test_quintic_trajectory_from_0p01,
               test_example_64x256_band_and_update_rms,
               test_transpose_equivariance,
               test_momentum_three_step_closed_form,
               test_ema_and_accumulating_forms_give_the_same_update,
               test_update_rms_of_exact_polar_factor,
               test_zero_gradient_gives_pure_decay_product,
               test_apply_superposition,
               test_converged_output_is_the_svd_polar_factor):
        try:
            fn()
        except (AssertionError, ValueError, FloatingPointError):
            fails.append(fn.__name__)
    return fails


def _planted_ns(variant):
    """A Newton-Schulz with one plausible mistake planted in it."""
    def ns(N, steps=5, coeffs=O.QUINTIC, eps=O.EPS):
        X = np.array(N, dtype=np.float64)
        a, b, c = coeffs
        tall = X.shape[0] > X.shape[1]
        if tall:
            X = X.T
        if variant == "spectral_instead_of_frobenius":
            X = X / (np.linalg.norm(X, 2) + eps)
        else:
            X = X / (math.sqrt(np.sum(X * X)) + eps)
        for _ in range(steps):
            A = X @ X.T
            if variant == "wrong_sign_b":
                X = a * X + (-b * A + c * (A @ A)) @ X
            elif variant == "dropped_c":
                X = a * X + (b * A) @ X
            elif variant == "square_instead_of_cube":
                X = a * X + b * A + c * (A @ A) @ X if X.shape[0] == X.shape[1] else a * X + (b * A) @ X
            else:
                X = a * X + (b * A + c * (A @ A)) @ X
        if variant == "output_left_transposed":
            return X
        return X.T if tall else X
    return ns


@pytest.mark.parametrize("variant", ["wrong_sign_b", "dropped_c", "spectral_instead_of_frobenius",
                                     "output_left_transposed", "square_instead_of_cube"])
def test_planted_newton_schulz_mistakes_are_caught(monkeypatch, variant):
    monkeypatch.setattr(O, "newton_schulz", _planted_ns(variant))
    assert _run_pins(), f"no pin caught planted mistake {variant}"


def _m_without_one_minus_beta(M, G, beta=O.BETA, nesterov=True):
    M2 = beta * np.asarray(M, float) + np.asarray(G, float)
    return M2, ((1 - beta) * np.asarray(G, float) + beta * M2) if nesterov else M2.copy()


def _m_nesterov_dropped(M, G, beta=O.BETA, nesterov=True):
    M2 = beta * np.asarray(M, float) + (1 - beta) * np.asarray(G, float)
    return M2, M2.copy()


def _m_nesterov_on_old_momentum(M, G, beta=O.BETA, nesterov=True):
    M0 = np.asarray(M, float)
    M2 = beta * M0 + (1 - beta) * np.asarray(G, float)
    return M2, ((1 - beta) * np.asarray(G, float) + beta * M0) if nesterov else M2.copy()


def _s_min_dim(m, n, mode=O.SCALE_MATCH_RMS, coeff=0.2):
    if mode == O.SCALE_MATCH_RMS:
        return coeff * math.sqrt(min(m, n))
    return math.sqrt(max(1.0, m / n)) if mode == O.SCALE_ORIGINAL else 1.0


def _a_decay_after_update(W, Ot, lr, weight_decay, mode=O.SCALE_MATCH_RMS, coeff=0.2):
    wd = weight_decay
    W = np.asarray(W, float)
    s = O.scale_factor(W.shape[0], W.shape[1], mode, coeff)
    return (1.0 - lr * wd) * (W - lr * s * np.asarray(Ot, float))


@pytest.mark.parametrize("attr,fn", [("momentum", _m_without_one_minus_beta),
                                     ("momentum", _m_nesterov_dropped),
                                     ("momentum", _m_nesterov_on_old_momentum),
                                     ("scale_factor", _s_min_dim),
                                     ("apply_update", _a_decay_after_update)])
def test_planted_momentum_and_apply_mistakes_are_caught(monkeypatch, attr, fn):
    monkeypatch.setattr(O, attr, fn)
    assert _run_pins(), f"no pin caught planted mistake {fn.__name__}"
