"""Pins of the fp64 SOAP oracle to facts the pages and mathematics fix.

"LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable Training"
(section 11), "初探优化器（一）：从SGD到SOAP-Muon" (section 6) and "Reading
notes on SOAP, Muon and higher-order optimizers" (section 2) fix, without
going through the oracle's own recurrences:

* the statistics after a few steps are explicit weighted sums of G G^T and
  G^T G;
* QR of the worked 2x2 matrix [[3, 0], [4, 5]] by hand, and of random
  matrices by classical Gram-Schmidt (a different algorithm);
* repeated power iteration plus QR on fixed statistics converges to the
  eigenvectors numpy's eigendecomposition returns, largest first;
* with those bases for a single gradient, no moving averages and a
  sign-like Adam step, the direction is the polar factor U V^T of an SVD;
* in the eigenbasis of L = G G^T the eigenvalues are the row sums of the
  squared rotated gradient, and those of R the column sums;
* a refresh changes the coordinates of the first moment, not the matrix it
  stands for;
* with both bases the identity the step is the AdamW step.

The last test plants plausible mistakes in the oracle (on the CPU) and checks
that at least one pin catches each.
"""

import numpy as np
import pytest

from oracle import adamw as A
from oracle import soap as S


def rng(seed):
    return np.random.default_rng(seed)


def spd_with_spectrum(n, lam, seed):
    Q, _ = np.linalg.qr(rng(seed).standard_normal((n, n)))
    return (Q * lam[None, :]) @ Q.T


def with_singular_values(m, n, sigma, seed):
    r = rng(seed)
    U, _ = np.linalg.qr(r.standard_normal((m, m)))
    V, _ = np.linalg.qr(r.standard_normal((n, n)))
    k = min(m, n)
    return (U[:, :k] * sigma[None, :]) @ V[:, :k].T


# --------------------------------------------------------------------- pins

def pin_statistics_weighted_sum(mod):
    r = rng(3)
    b = 0.8
    Gs = [r.standard_normal((5, 7)) for _ in range(3)]
    L, R = np.zeros((5, 5)), np.zeros((7, 7))
    for G in Gs:
        L, R = mod.statistics(L, R, G, b)
    wl = (1 - b) * sum(b ** (2 - k) * Gs[k] @ Gs[k].T for k in range(3))
    wr = (1 - b) * sum(b ** (2 - k) * Gs[k].T @ Gs[k] for k in range(3))
    np.testing.assert_allclose(L, wl, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(R, wr, rtol=1e-13, atol=1e-14)


def pin_qr_worked_example(mod):
    # [[3,0],[4,5]]: first column (3,4)/5; the second, (0,5) minus its
    # projection 4*(0.6,0.8), is (-2.4,1.8) of length 3
    Q, R = mod.qr_nonneg(np.array([[3.0, 0.0], [4.0, 5.0]]))
    np.testing.assert_allclose(Q, [[0.6, -0.8], [0.8, 0.6]], atol=1e-15)
    np.testing.assert_allclose(R, [[5.0, 4.0], [0.0, 3.0]], atol=1e-14)


def gram_schmidt(A):
    A = np.array(A, dtype=np.float64)
    n = A.shape[1]
    Q = np.zeros_like(A)
    for j in range(n):
        v = A[:, j].copy()
        for i in range(j):
            v -= (Q[:, i] @ A[:, j]) * Q[:, i]
        Q[:, j] = v / np.linalg.norm(v)
    return Q


def pin_qr_gram_schmidt(mod):
    for seed, n in ((4, 6), (5, 9)):
        A_ = rng(seed).standard_normal((n, n)) + 3 * np.eye(n)
        Q, R = mod.qr_nonneg(A_)
        np.testing.assert_allclose(Q, gram_schmidt(A_), atol=1e-12)
        assert np.all(np.diag(R) >= 0)
        np.testing.assert_allclose(np.tril(R, -1), 0, atol=1e-13)


def pin_power_iteration_converges(mod):
    n = 8
    lam = 2.0 ** -np.arange(n)              # ratio 1/2 between neighbours
    Lm = spd_with_spectrum(n, lam, 6)
    Q = np.eye(n)
    for _ in range(120):
        Q = mod.power_qr(Lm, Q)
    w, U = np.linalg.eigh(Lm)
    U = U[:, ::-1]                          # largest first
    np.testing.assert_allclose(np.abs(np.sum(Q * U, axis=0)), 1.0, atol=1e-12)
    np.testing.assert_allclose(Q.T @ Lm @ Q, np.diag(lam), atol=1e-13)


def converged_bases(mod, G, iters=200):
    m, n = G.shape
    L, R = mod.statistics(np.zeros((m, m)), np.zeros((n, n)), G, 0.0)
    QL, QR = np.eye(m), np.eye(n)
    for _ in range(iters):
        QL, QR, _ = mod.refresh(L, R, QL, QR, np.zeros((m, n)))
    return L, R, QL, QR


def pin_polar_limit(mod):
    # [NOTES] 2: Q_L = U, Q_R = V, EMA off, Adam step ~ sign -> D = U V^T
    n = 6
    sigma = 1.6 ** -np.arange(n) * 4.0
    G = with_singular_values(n, n, sigma, 7)
    _, _, QL, QR = converged_bases(mod, G)
    # eps keeps the round-off left off the diagonal of Gbar (~1e-16) from
    # being normalized to a unit step; its effect on the diagonal is eps/sigma
    D, _, _ = mod.precondition(G, QL, QR, np.zeros((n, n)), np.zeros((n, n)), 1, 0.0, 0.0, 1e-7)
    U, _, Vt = np.linalg.svd(G)
    np.testing.assert_allclose(D, U @ Vt, atol=1e-6)


def pin_row_column_sums(mod):
    # [ZH] 6.1: in the eigenbasis, eig(L)_i = sum_j Gbar_ij^2, eig(R)_j = sum_i Gbar_ij^2
    m, n = 5, 7
    G = with_singular_values(m, n, 1.7 ** -np.arange(m) * 3.0, 8)
    L, R, QL, QR = converged_bases(mod, G, iters=300)
    Gbar = QL.T @ G @ QR
    np.testing.assert_allclose(np.diag(QL.T @ L @ QL), np.sum(Gbar ** 2, axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(np.diag(QR.T @ R @ QR), np.sum(Gbar ** 2, axis=0), rtol=1e-10, atol=1e-12)


def pin_refresh_keeps_moment(mod):
    # [GUIDE] 11.1: the refresh changes the coordinates of the first moment only
    r = rng(9)
    m, n = 6, 4
    L = spd_with_spectrum(m, r.uniform(0.5, 2, m), 10)
    R = spd_with_spectrum(n, r.uniform(0.5, 2, n), 11)
    QL = np.linalg.qr(r.standard_normal((m, m)))[0]
    QR = np.linalg.qr(r.standard_normal((n, n)))[0]
    Mbar = r.standard_normal((m, n))
    QLn, QRn, Mn = mod.refresh(L, R, QL, QR, Mbar)
    np.testing.assert_allclose(QLn @ Mn @ QRn.T, QL @ Mbar @ QR.T, atol=1e-13)
    # the new bases are the QR factors of S Q
    np.testing.assert_allclose(QLn.T @ QLn, np.eye(m), atol=1e-13)
    assert np.allclose(np.tril(QLn.T @ (L @ QL), -1), 0, atol=1e-12)
    assert np.allclose(np.tril(QRn.T @ (R @ QR), -1), 0, atol=1e-12)


def pin_identity_is_adamw(mod):
    # [GUIDE] 11.2: both bases identity -> the layer is AdamW
    r = rng(12)
    m, n = 4, 5
    W = r.standard_normal((m, n))
    st = mod.init_state(m, n, max_dim=0)
    th, mm, vv = W.copy(), np.zeros((m, n)), np.zeros((m, n))
    for t in range(1, 4):
        G = r.standard_normal((m, n)) * 10 ** r.uniform(-3, 1)
        W, _ = mod.soap_step(W, G, st, lr=0.01, weight_decay=0.1, beta1=0.9, beta2=0.99, eps=1e-8)
        th, mm, vv = A.adamw_step(th, G, mm, vv, t, 0.01, 0.9, 0.99, 1e-8, 0.1)
        np.testing.assert_allclose(W, th, rtol=1e-13, atol=1e-15)


def pin_one_sided(mod):
    # an axis over max_dim keeps the identity: the step equals a two-sided
    # step whose column statistic is never refreshed away from I
    r = rng(13)
    m, n = 4, 9
    st = mod.init_state(m, n, max_dim=5)
    assert st.R is None and st.L is not None
    W = r.standard_normal((m, n))
    G = r.standard_normal((m, n))
    W1, D = mod.soap_step(W, G, st, lr=0.1, freq=1)
    QL = S.power_qr((1 - S.BETA_S) * G @ G.T, np.eye(m))
    Gbar = QL.T @ G
    want = QL @ (Gbar / (np.abs(Gbar) + S.EPS))      # t = 1: m_hat = Gbar, v_hat = Gbar^2
    np.testing.assert_allclose(D, want, atol=1e-12)


PINS = [pin_statistics_weighted_sum, pin_qr_worked_example, pin_qr_gram_schmidt, pin_power_iteration_converges,
        pin_polar_limit, pin_row_column_sums, pin_refresh_keeps_moment, pin_identity_is_adamw, pin_one_sided]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(S)


def test_refresh_schedule():
    # reading 3: refreshes on t = 1, 1+f, ...; the bases stay fixed in between
    r = rng(14)
    m, n = 5, 6
    st = S.init_state(m, n, max_dim=64)
    W = r.standard_normal((m, n))
    seen = []
    for t in range(1, 8):
        before = st.QL.copy()
        W, _ = S.soap_step(W, r.standard_normal((m, n)), st, lr=0.01, freq=3)
        seen.append(not np.array_equal(before, st.QL))
    assert seen == [True, False, False, True, False, False, True]


def test_zero_gradient_is_decay_only():
    st = S.init_state(3, 4, max_dim=8)
    W = rng(15).standard_normal((3, 4))
    W1, D = S.soap_step(W, np.zeros((3, 4)), st, lr=0.5, weight_decay=0.2)
    assert np.all(D == 0)
    np.testing.assert_allclose(W1, 0.9 * W, rtol=1e-15)


# ------------------------------------------------------- planted mistakes

class _Mutant:
    """The oracle with one function replaced."""

    def __init__(self, **over):
        self.__dict__.update({k: getattr(S, k) for k in dir(S) if not k.startswith("__")})
        self.__dict__.update(over)


def _mut_stats_swapped(L, R, G, b):
    # the averaging weights exchanged
    G = np.asarray(G, float)
    L = None if L is None else (1 - b) * L + b * (G @ G.T)
    R = None if R is None else (1 - b) * R + b * (G.T @ G)
    return L, R


def _mut_qr_no_sign(A_):
    return np.linalg.qr(np.asarray(A_, float))


def _mut_power_transposed(Sm, Q):
    return S.qr_nonneg(np.asarray(Q, float) @ np.asarray(Sm, float))[0]


def _mut_refresh_wrong_rotation(L, R, QL, QR, Mbar):
    QLn = S.power_qr(L, QL) if L is not None else QL
    QRn = S.power_qr(R, QR) if R is not None else QR
    return QLn, QRn, Mbar          # moment not carried into the new basis


def _mut_no_bias_correction(G, QL, QR, Mbar, Vbar, t, b1, b2, eps):
    Gbar = QL.T @ G @ QR
    Mbar = b1 * Mbar + (1 - b1) * Gbar
    Vbar = b2 * Vbar + (1 - b2) * Gbar * Gbar
    return QL @ (Mbar / (np.sqrt(Vbar) + eps)) @ QR.T, Mbar, Vbar


def _mut_back_rotation_transposed(G, QL, QR, Mbar, Vbar, t, b1, b2, eps):
    D, Mbar, Vbar = S.precondition(G, QL, QR, Mbar, Vbar, t, b1, b2, eps)
    Dbar = QL.T @ D @ QR
    return QL.T @ Dbar @ QR, Mbar, Vbar


MUTANTS = {
    "statistics weights exchanged": dict(statistics=_mut_stats_swapped),
    "QR without the sign convention": dict(qr_nonneg=_mut_qr_no_sign),
    "power step Q S instead of S Q": dict(power_qr=_mut_power_transposed),
    "moment not re-rotated": dict(refresh=_mut_refresh_wrong_rotation),
    "no bias correction": dict(precondition=_mut_no_bias_correction),
    "back rotation transposed": dict(precondition=_mut_back_rotation_transposed),
}


def _soap_step_of(mod):
    # soap_step looks its helpers up in the oracle module; rebuild it over
    # the mutant's functions
    def step(W, G, st, lr, weight_decay=0.0, beta1=S.BETA1, beta2=S.BETA2, eps=S.EPS, beta_s=S.BETA_S,
             freq=S.FREQ):
        st.t += 1
        st.L, st.R = mod.statistics(st.L, st.R, G, beta_s)
        if (st.t - 1) % freq == 0:
            st.QL, st.QR, st.Mbar = mod.refresh(st.L, st.R, st.QL, st.QR, st.Mbar)
        D, st.Mbar, st.Vbar = mod.precondition(G, st.QL, st.QR, st.Mbar, st.Vbar, st.t, beta1, beta2, eps)
        return (1 - lr * weight_decay) * W - lr * D, D
    return step


def _refresh_of(mod):
    def refresh(L, R, QL, QR, Mbar):
        QLn = mod.power_qr(L, QL) if L is not None else QL
        QRn = mod.power_qr(R, QR) if R is not None else QR
        if L is not None:
            Mbar = QLn.T @ (QL @ Mbar)
        if R is not None:
            Mbar = (Mbar @ QR.T) @ QRn
        return QLn, QRn, Mbar
    return refresh


def _power_of(mod):
    return lambda Sm, Q: mod.qr_nonneg(np.asarray(Sm, float) @ np.asarray(Q, float))[0]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    over = dict(MUTANTS[name])
    mod = _Mutant(**over)
    # rebuild the composite functions over the mutant's parts, keeping any
    # part the mutant replaces itself
    if "power_qr" not in over:
        mod.power_qr = _power_of(mod)
    if "refresh" not in over:
        mod.refresh = _refresh_of(mod)
    mod.soap_step = _soap_step_of(mod)
    caught = 0
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches: {name}"
