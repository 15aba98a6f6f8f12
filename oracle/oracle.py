"""Plain fp64 CPU oracle for one Muon optimizer step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in the package entry module and the ``cpu_baseline`` leg of the benchmark may
import or call anything here.  The GPU library never routes through it, and
the two share no code, headers, constants or helpers: the only thing both
sides see is the seeded input generator, which holds none of the method's
arithmetic.

Everything is NumPy float64, one matrix at a time, with no blocking, fusion or
rounding emulation.  Each function states the passage it follows.  Sources
(the "pages"):

* [NOTES]   "Reading notes on SOAP, Muon and higher-order optimizers"
            (jianyuh.github.io), section 1 "AdamW vs. SOAP vs. Muon".
* [PREPRINT] "SOAP, Muon, and Beyond: Pushing LLM Pretraining Scales"
            (agihunt.info summary), limitations paragraph (the epsilon value).
* [GUIDE]   "LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
            Training", sections 11.3 (momentum / Nesterov), 11.4
            (Newton-Schulz equations), 11.5 (shape scaling and decoupled
            decay).
* [LESSON]  "Matrix optimizers: K-FAC, Shampoo and Muon" (Lesson 12),
            subsections "Newton-Schulz: UV^T with matrix products only"
            (Lemma 3 and its three-step algorithm) and "Muon" (steps 1-4 and
            the remark on the moving-average form of the momentum).
* [ZH]      "初探优化器（一）：从SGD到SOAP-Muon", section 4.3 (the iteration
            and its coefficient sets).

Readings taken where the pages leave a step open are listed next to the code
that takes them.

Pin status: every function here is pinned by the CPU tests against values
the pages print (worked 2x2 example, scalar trajectories, the 64x256 band and
update RMS), against closed forms (Lemma 3 via an SVD, the exact polar factor,
the EMA geometric sum, the decay product) and against invariants (transpose
equivariance, scale invariance, odd symmetry); the checker
``relative_frobenius_error`` is pinned to hand-computed values on integer
matrices.  No function is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Jordan's quintic coefficients, [GUIDE] 11.4 and [LESSON] "Muon's quintic".
QUINTIC = (3.4445, -4.7750, 2.0315)
# The classical cubic iteration, [LESSON] "The cubic (classical) iteration".
CUBIC = (1.5, -0.5, 0.0)
# A convergent quintic quoted in [ZH] 4.3 (p(1) = 1, slope 2 at zero).
TRACK3 = (2.0, -1.5, 0.5)
# Muon's epsilon: [PREPRINT] (1e-7 for Muon) and the default of [GUIDE] 11.4.
EPS = 1e-7
# Default momentum coefficient, [LESSON] "Muon" (0.95 by default).
BETA = 0.95

SCALE_MATCH_RMS = 0
SCALE_ORIGINAL = 1
SCALE_NONE = 2


def _f64(x) -> np.ndarray:
    return np.array(x, dtype=np.float64, copy=True)


def momentum(mom, grad, beta: float = BETA, nesterov: bool = True):
    """One momentum update; returns ``(new_momentum, ns_input)``.

    Moving average M_t = beta*M_{t-1} + (1-beta)*G_t as written in [NOTES]
    section 1.  [GUIDE] 11.3 and [LESSON] "Muon" step 1 write the
    accumulating form B_t = beta*B_{t-1} + G_t; [LESSON] notes that the
    moving average only rescales that buffer (M = (1-beta)*B from zero), and
    Newton-Schulz divides by the Frobenius norm, so the orthogonalized output
    is the same up to epsilon.

    Nesterov blend: [GUIDE] 11.3 and [LESSON] step 2 give
    N = G_t + beta*B_t in the accumulating form.  Multiplying by (1-beta)
    gives the moving-average form used here,
    N = (1-beta)*G_t + beta*M_t  (reading: the pages never write this form;
    it is the exact image of theirs under M = (1-beta)*B).
    Without Nesterov, N = M_t.  Nesterov is the default ([ZH] 1.3 calls it
    Muon's default).
    """
    M = _f64(mom)
    G = _f64(grad)
    if M.shape != G.shape:
        raise ValueError("momentum and gradient shapes differ")
    if not (0.0 <= beta < 1.0):
        raise ValueError("beta must lie in [0, 1)")
    M_new = beta * M + (1.0 - beta) * G
    if nesterov:
        N = (1.0 - beta) * G + beta * M_new
    else:
        N = M_new.copy()
    return M_new, N


def frobenius_sumsq(N) -> float:
    """Sum of squares of all entries; its square root is the Frobenius norm
    that normalizes the Newton-Schulz input ([GUIDE] 11.4, X_0 equation)."""
    X = _f64(N)
    return float(np.sum(X * X))


def is_tall(rows: int, cols: int) -> bool:
    """Tall matrices are worked on transposed so that the Gram matrix is the
    smaller one: strictly rows > cols ([LESSON] algorithm step 2, [GUIDE]
    11.4).  Square matrices are not transposed."""
    return rows > cols


def newton_schulz(N, steps: int = 5, coeffs=QUINTIC, eps: float = EPS):
    """Approximate polar factor of ``N`` by ``steps`` Newton-Schulz steps.

    [LESSON] "Newton-Schulz: UV^T with matrix products only", algorithm:
      1. normalize X_0 = N / (||N||_F + eps)   (eps added to the norm, not to
         the sum of squares: [GUIDE] 11.4 X_0 equation);
      2. if rows > cols, work on the transpose so X X^T is the smaller Gram;
      3. repeat: A = X X^T, X <- a X + (b A + c A^2) X   ([GUIDE] 11.4;
         [LESSON] Lemma 3 writes the same step as aX + b(XX^T)X + c(XX^T)^2 X).
    The output has the input's orientation.  Coefficients are the same at
    every step.
    """
    X = _f64(N)
    if X.ndim != 2:
        raise ValueError("Newton-Schulz needs a 2-D matrix")
    if steps < 0:
        raise ValueError("steps must be >= 0")
    a, b, c = (float(v) for v in coeffs)
    transposed = is_tall(*X.shape)
    if transposed:
        X = X.T.copy()
    X = X / (math.sqrt(frobenius_sumsq(X)) + eps)
    for _ in range(steps):
        A = X @ X.T
        poly = b * A + c * (A @ A)
        X = a * X + poly @ X
    return X.T.copy() if transposed else X


def scale_factor(rows: int, cols: int, mode: int = SCALE_MATCH_RMS,
                 coeff: float = 0.2) -> float:
    """Shape factor s of the update ([GUIDE] 11.5; [LESSON] "Muon" step 4).

    * MATCH_RMS: s = coeff*sqrt(max(m, n)); coeff = 0.2 gives the
      update-RMS match to AdamW ([GUIDE] 11.5, [LESSON] "Update size").
      Reading: [NOTES] section 3 names a correction factor
      sqrt((1-beta)/(1+beta)); it is accepted here as a value of ``coeff``.
    * ORIGINAL: s = sqrt(max(1, m/n)) (Jordan's choice).
    * NONE: s = 1.
    """
    if mode == SCALE_MATCH_RMS:
        return float(coeff) * math.sqrt(max(rows, cols))
    if mode == SCALE_ORIGINAL:
        return math.sqrt(max(1.0, rows / cols))
    if mode == SCALE_NONE:
        return 1.0
    raise ValueError("unknown scale mode")


def apply_update(weight, ortho, lr: float, weight_decay: float,
                 mode: int = SCALE_MATCH_RMS, coeff: float = 0.2):
    """W_t = (1 - lr*wd) W_{t-1} - lr * s * O_t  ([GUIDE] 11.5 update
    equation; [LESSON] "Muon" step 4).  Both terms read W_{t-1}."""
    W = _f64(weight)
    O = _f64(ortho)
    if W.shape != O.shape:
        raise ValueError("weight and update shapes differ")
    s = scale_factor(W.shape[0], W.shape[1], mode, coeff)
    return (1.0 - lr * weight_decay) * W - lr * s * O


def muon_step(weight, mom, grad, *, beta: float = BETA, nesterov: bool = True,
              steps: int = 5, coeffs=QUINTIC, eps: float = EPS,
              lr: float = 3e-4, weight_decay: float = 0.1,
              mode: int = SCALE_MATCH_RMS, coeff: float = 0.2):
    """One full step for one matrix: momentum, orthogonalize, apply
    ([LESSON] "Muon" steps 1-4 in that order).

    Returns ``(new_weight, new_momentum, ortho, sumsq)`` where ``sumsq`` is
    the sum of squares of the Newton-Schulz input.
    """
    M_new, N = momentum(mom, grad, beta, nesterov)
    sumsq = frobenius_sumsq(N)
    O = newton_schulz(N, steps, coeffs, eps)
    W_new = apply_update(weight, O, lr, weight_decay, mode, coeff)
    return W_new, M_new, O, sumsq


def relative_frobenius_error(got, want) -> float:
    """||got - want||_F / ||want||_F, entries paired by position; ||got||_F
    when ``want`` is zero.  This is the measure the parity tolerances are
    stated in (relative Frobenius error).  Both arguments must have the same
    shape: NumPy would otherwise broadcast (n, 1) against (1, n)."""
    g = _f64(got)
    w = _f64(want)
    if g.shape != w.shape:
        raise ValueError(f"shapes differ: {g.shape} vs {w.shape}")
    den = math.sqrt(float(np.sum(w * w)))
    num = math.sqrt(float(np.sum((g - w) ** 2)))
    if den == 0.0:
        return num
    return num / den
