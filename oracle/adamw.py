"""Plain fp64 CPU oracle for the AdamW step that covers the parameters Muon
does not (embeddings, output head, norms, biases).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite and the
benchmark's ``cpu_baseline`` leg may import or call anything here; the GPU
library shares no code with it.

Source ("the pages"):

* [GUIDE] "LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
  Training", section 5 "Adam, line by line" (the two moving averages, bias
  correction by the accumulated mass 1 - beta^t, epsilon outside the square
  root, the constant-gradient limit), section 6 (decoupled weight decay as
  one combined expression, the decay product, the default hyperparameters of
  its from-scratch optimizer) and section 6.2 (a missing gradient is not a
  zero gradient).

Everything is NumPy float64, elementwise, with no fusion or rounding
emulation.

Pin status: pinned by the CPU tests against the guide's closed forms (the
constant-gradient limit m_hat = g, v_hat = g^2, the geometric-sum mass
(1 - beta1^t), the decay product with a zero gradient), against a direct
weighted sum of a gradient sequence, and against the exact affine split of
the decoupled decay.  Not "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Defaults of the from-scratch optimizer in [GUIDE] section 6.
BETA1 = 0.9
BETA2 = 0.999
EPS = 1e-8


def _f64(x) -> np.ndarray:
    return np.array(x, dtype=np.float64, copy=True)


def adamw_step(param, grad, exp_avg, exp_avg_sq, step: int, lr: float, beta1: float = BETA1,
               beta2: float = BETA2, eps: float = EPS, weight_decay: float = 0.0):
    """One AdamW step for one tensor; returns ``(param, exp_avg, exp_avg_sq)``.

    In the order of [GUIDE] sections 5 and 6:
      m_t = beta1*m_{t-1} + (1-beta1)*g_t
      v_t = beta2*v_{t-1} + (1-beta2)*g_t^2
      m_hat = m_t / (1 - beta1^t),  v_hat = v_t / (1 - beta2^t)
      theta_t = (1 - lr*wd)*theta_{t-1} - lr * m_hat / (sqrt(v_hat) + eps)
    Epsilon is added after the square root, as in Adam and PyTorch's AdamW
    ([GUIDE] section 5).  ``step`` is t, counted from 1 for the first update
    of this tensor; a step with no gradient is not a call at all ([GUIDE]
    6.2), while an all-zero gradient is a normal call.
    """
    theta = _f64(param)
    g = _f64(grad)
    m = _f64(exp_avg)
    v = _f64(exp_avg_sq)
    if not (theta.shape == g.shape == m.shape == v.shape):
        raise ValueError("parameter, gradient and state shapes differ")
    if int(step) != step or step < 1:
        raise ValueError("step counts updates from 1")
    if not (0.0 <= beta1 < 1.0 and 0.0 <= beta2 < 1.0):
        raise ValueError("betas must lie in [0, 1)")
    if not (math.isfinite(lr) and math.isfinite(weight_decay) and math.isfinite(eps) and eps >= 0.0):
        raise ValueError("lr, weight_decay and eps must be finite, eps >= 0")
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    theta = (1.0 - lr * weight_decay) * theta - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v
