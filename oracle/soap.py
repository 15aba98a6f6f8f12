"""Plain fp64 CPU oracle for the SOAP step: Adam run in the eigenbasis of
Shampoo's row and column statistics.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite and the
benchmark's ``cpu_baseline`` leg may import or call anything here; the GPU
library shares no code with it.

Sources ("the pages"):

* [GUIDE] "LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
  Training", section 11.1 "SOAP: Adam in Shampoo's eigenbasis" (the moving
  row and column statistics, the refresh every f steps, the first moment kept
  in the rotated basis and carried exactly into a new basis, the second moment
  estimated in the active basis, the bias-corrected direction, the rotation
  back and the decoupled decay) and section 11.2 (refresh by power iteration
  plus QR; identity basis on very large axes; both bases identity reduces the
  layer to AdamW).
* [ZH] "初探优化器（一）：从SGD到SOAP-Muon", section 6.2 (the five steps of
  one SOAP update; one power-iteration step plus a QR factorization as the
  cheap stand-in for an eigendecomposition) and section 6.1 (in the
  eigenbasis, the eigenvalues of L and R are the row and column sums of the
  squared rotated gradient).
* [NOTES] "Reading notes on SOAP, Muon and higher-order optimizers", section
  2 (with the singular vectors as bases, no moving averages and a sign-like
  Adam step, SOAP's direction is the polar factor U V^T) and section 4 (fold
  the current gradient into the basis refresh).

Readings where the pages leave a step open (each also noted at its code):

1. The first moment lives in the rotated basis and is re-expressed on each
   refresh ([GUIDE] 11.1).  [ZH] 6.2 instead rotates a parameter-space
   momentum every step; the two are equal in exact arithmetic because the
   map is linear.
2. A refresh is one power-iteration step from the current basis followed by
   a QR factorization, Q <- qr(S Q), with the triangular factor's diagonal
   made non-negative so that Q is unique for full-rank S Q.  Bases start as
   the identity.
3. At step t the statistics take G_t first; the bases are refreshed on steps
   t = 1, 1 + f, 1 + 2f, ... from those statistics (the current gradient
   folded in, [NOTES] 4); then G_t is rotated in the active basis.
4. Epsilon is added after the square root, and both moments are
   bias-corrected by 1 - beta^t ([GUIDE] 11.1 writes the hats, as in Adam).
5. An axis longer than ``max_dim`` keeps the identity basis and no statistic
   ([GUIDE] 11.2).

Everything is NumPy float64, one matrix at a time.  numpy's QR (LAPACK's
Householder factorization) serves as the library primitive for step 2.

Pin status: pinned by the CPU tests against a worked 2x2 QR, classical
Gram-Schmidt, the statistics' explicit weighted sums, convergence of the
repeated refresh to numpy's eigendecomposition, the polar factor from an SVD
(the unification limit), the row/column-sum identity, exact invariance of the
parameter-space first moment under a refresh, and the AdamW oracle (both
bases identity).  Not "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Defaults: Adam's of [GUIDE] section 6; the statistics' average 0.9 is the
# value [ZH] 7.2 reports for the SOAP-Muon records; f = 10 is the guide's
# "e.g., every 10 steps" staleness example ([NOTES] 4).
BETA1 = 0.9
BETA2 = 0.999
EPS = 1e-8
BETA_S = 0.9
FREQ = 10


def _f64(x) -> np.ndarray:
    return np.array(x, dtype=np.float64, copy=True)


def statistics(L, R, G, beta_s: float):
    """[GUIDE] 11.1, [ZH] 6.2 step 1: L <- b L + (1-b) G G^T,
    R <- b R + (1-b) G^T G.  A side passed as None stays None."""
    G = _f64(G)
    if L is not None:
        L = beta_s * _f64(L) + (1.0 - beta_s) * (G @ G.T)
    if R is not None:
        R = beta_s * _f64(R) + (1.0 - beta_s) * (G.T @ G)
    return L, R


def qr_nonneg(A):
    """QR factorization A = Q R with R's diagonal made non-negative
    (reading 2).  Returns (Q, R)."""
    Q, R = np.linalg.qr(_f64(A))
    d = np.where(np.diag(R) < 0.0, -1.0, 1.0)
    return Q * d[None, :], R * d[:, None]


def power_qr(S, Q):
    """One power-iteration step plus QR ([GUIDE] 11.2, [ZH] 6.2 step 2)."""
    return qr_nonneg(_f64(S) @ _f64(Q))[0]


def refresh(L, R, QL, QR, Mbar):
    """New bases from the statistics, and the rotated first moment carried
    into them ([GUIDE] 11.1): Mbar_new = QL_new^T QL_old Mbar QR_old^T QR_new.
    A side whose statistic is None keeps its (identity) basis."""
    QLn = power_qr(L, QL) if L is not None else QL
    QRn = power_qr(R, QR) if R is not None else QR
    Mbar = _f64(Mbar)
    if L is not None:
        Mbar = QLn.T @ (QL @ Mbar)
    if R is not None:
        Mbar = (Mbar @ QR.T) @ QRn
    return QLn, QRn, Mbar


def precondition(G, QL, QR, Mbar, Vbar, t: int, beta1: float, beta2: float, eps: float):
    """[GUIDE] 11.1 between refreshes: rotate, Adam in the rotated basis,
    rotate back.  Returns (D, Mbar, Vbar)."""
    G = _f64(G)
    Gbar = QL.T @ G @ QR
    Mbar = beta1 * _f64(Mbar) + (1.0 - beta1) * Gbar
    Vbar = beta2 * _f64(Vbar) + (1.0 - beta2) * Gbar * Gbar
    m_hat = Mbar / (1.0 - beta1 ** t)
    v_hat = Vbar / (1.0 - beta2 ** t)
    Dbar = m_hat / (np.sqrt(v_hat) + eps)
    return QL @ Dbar @ QR.T, Mbar, Vbar


@dataclass
class State:
    """Per-matrix SOAP state: statistics, bases, rotated moments, step."""
    L: np.ndarray | None
    R: np.ndarray | None
    QL: np.ndarray
    QR: np.ndarray
    Mbar: np.ndarray
    Vbar: np.ndarray
    t: int = 0
    extra: dict = field(default_factory=dict)


def init_state(m: int, n: int, max_dim: int) -> State:
    """Zero statistics and moments, identity bases; an axis longer than
    ``max_dim`` gets no statistic (reading 5)."""
    L = np.zeros((m, m)) if m <= max_dim else None
    R = np.zeros((n, n)) if n <= max_dim else None
    return State(L, R, np.eye(m), np.eye(n), np.zeros((m, n)), np.zeros((m, n)))


def soap_step(W, G, st: State, lr: float, weight_decay: float = 0.0, beta1: float = BETA1,
              beta2: float = BETA2, eps: float = EPS, beta_s: float = BETA_S, freq: int = FREQ):
    """One SOAP update of W (m x n) with gradient G; advances ``st`` in place
    and returns (W_new, D).  Order of reading 3."""
    if not (0.0 <= beta1 < 1.0 and 0.0 <= beta2 < 1.0 and 0.0 <= beta_s < 1.0):
        raise ValueError("betas must lie in [0, 1)")
    if freq < 1 or not (math.isfinite(eps) and eps >= 0.0):
        raise ValueError("freq >= 1 and a finite eps >= 0 are required")
    st.t += 1
    st.L, st.R = statistics(st.L, st.R, G, beta_s)
    if (st.t - 1) % freq == 0:
        st.QL, st.QR, st.Mbar = refresh(st.L, st.R, st.QL, st.QR, st.Mbar)
    D, st.Mbar, st.Vbar = precondition(G, st.QL, st.QR, st.Mbar, st.Vbar, st.t, beta1, beta2, eps)
    W = (1.0 - lr * weight_decay) * _f64(W) - lr * D
    return W, D
