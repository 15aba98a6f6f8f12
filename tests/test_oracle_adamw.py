"""Pins of the fp64 AdamW oracle to facts the guide and mathematics fix.

"LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable Training",
sections 5 and 6, give closed forms that do not go through the recurrence
the oracle runs:

* a constant gradient g from zero state gives m_hat = g and v_hat = g^2 at
  every step, so each step moves the parameter by -lr*g/(|g|+eps);
* the first moment after t steps is the geometric mass (1 - beta1^t) times
  a constant gradient, and in general the weighted sum
  (1-beta1) * sum_k beta1^(t-k) g_k;
* with a zero gradient from zero state the parameter only decays, by the
  product of (1 - lr_t*wd);
* the decoupled decay enters as an exact affine term -lr*wd*theta.

The last tests plant plausible mistakes in the oracle (on the CPU) and check
that at least one pin catches each.
"""

import math

import numpy as np
import pytest

from oracle import adamw as A

RTOL = 1e-13


def rng(seed):
    return np.random.default_rng(seed)


def run(step_fn, theta0, grads, lrs, wd, beta1=A.BETA1, beta2=A.BETA2, eps=A.EPS):
    theta, m, v = theta0.copy(), np.zeros_like(theta0), np.zeros_like(theta0)
    out = []
    for t, (g, lr) in enumerate(zip(grads, lrs), start=1):
        theta, m, v = step_fn(theta, g, m, v, t, lr, beta1, beta2, eps, wd)
        out.append((theta, m, v))
    return out


# --------------------------------------------------------------------- pins

def pin_constant_gradient(step_fn):
    r = rng(1)
    g = r.standard_normal(257) * np.exp(r.uniform(-6, 3, 257))
    theta0 = r.standard_normal(257)
    lr = 1e-3
    states = run(step_fn, theta0, [g] * 12, [lr] * 12, 0.0)
    for t, (theta, m, v) in enumerate(states, start=1):
        # the raw first moment carries the mass (1 - beta1^t) of g
        np.testing.assert_allclose(m, (1 - A.BETA1 ** t) * g, rtol=RTOL, atol=0)
        np.testing.assert_allclose(v, (1 - A.BETA2 ** t) * g * g, rtol=RTOL, atol=0)
        # m_hat = g, v_hat = g^2: t identical steps of -lr*g/(|g|+eps)
        want = theta0 - t * lr * g / (np.abs(g) + A.EPS)
        np.testing.assert_allclose(theta, want, rtol=1e-12, atol=1e-15)


def pin_epsilon_outside_root(step_fn):
    # g = eps: the first step is lr * eps / (eps + eps) = lr/2; with eps under
    # the root it would be lr * eps / sqrt(eps^2 + eps), about 1e-4 * lr
    g = np.full(4, A.EPS)
    theta, _, _ = step_fn(np.zeros(4), g, np.zeros(4), np.zeros(4), 1, 1.0, A.BETA1, A.BETA2, A.EPS, 0.0)
    np.testing.assert_allclose(theta, -0.5, rtol=1e-12)


def pin_sign_step(step_fn):
    # |g| >> eps: the first step is a sign step of length lr
    g = np.array([1e3, -2e2, 7.0, -0.25])
    theta, _, _ = step_fn(np.ones(4), g, np.zeros(4), np.zeros(4), 1, 0.01, A.BETA1, A.BETA2, A.EPS, 0.0)
    np.testing.assert_allclose(theta, 1.0 - 0.01 * np.sign(g), rtol=1e-9)


def pin_weighted_sum(step_fn):
    # m_t and v_t against the explicit sums over a gradient sequence
    r = rng(2)
    T, n = 9, 33
    grads = [r.standard_normal(n) for _ in range(T)]
    b1, b2 = 0.8, 0.95
    states = run(step_fn, r.standard_normal(n), grads, [1e-2] * T, 0.0, b1, b2)
    m_sum = sum((1 - b1) * b1 ** (T - k) * grads[k - 1] for k in range(1, T + 1))
    v_sum = sum((1 - b2) * b2 ** (T - k) * grads[k - 1] ** 2 for k in range(1, T + 1))
    np.testing.assert_allclose(states[-1][1], m_sum, rtol=1e-12)
    np.testing.assert_allclose(states[-1][2], v_sum, rtol=1e-12)


def pin_decay_product(step_fn):
    # zero gradient from zero state: pure decay by prod(1 - lr_t * wd)
    r = rng(3)
    theta0 = r.standard_normal(20)
    lrs = list(np.linspace(1e-3, 5e-2, 15))
    wd = 0.7
    states = run(step_fn, theta0, [np.zeros(20)] * 15, lrs, wd)
    want = theta0 * np.prod([1 - lr * wd for lr in lrs])
    np.testing.assert_allclose(states[-1][0], want, rtol=1e-13)


def pin_affine_decay(step_fn):
    # the decay is -lr*wd*theta on top of the undecayed step, for any state
    r = rng(4)
    theta, g = r.standard_normal(50), r.standard_normal(50)
    m, v = r.standard_normal(50), r.uniform(0.1, 2.0, 50)
    lr, wd, t = 3e-2, 0.3, 5
    with_wd, _, _ = step_fn(theta, g, m, v, t, lr, A.BETA1, A.BETA2, A.EPS, wd)
    no_wd, _, _ = step_fn(theta, g, m, v, t, lr, A.BETA1, A.BETA2, A.EPS, 0.0)
    np.testing.assert_allclose(with_wd, no_wd - lr * wd * theta, rtol=1e-12, atol=1e-15)


PINS = [pin_constant_gradient, pin_epsilon_outside_root, pin_sign_step, pin_weighted_sum, pin_decay_product,
        pin_affine_decay]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_adamw_oracle_pin(pin):
    pin(A.adamw_step)


def test_adamw_invalid_hyperparameters_raise():
    z = np.zeros(3)
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, z, 0, 1e-3)
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, z, 1, 1e-3, beta1=1.0)
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, z, 1, 1e-3, beta2=-0.1)
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, z, 1, 1e-3, eps=-1e-8)
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, z, 1, float("nan"))
    with pytest.raises(ValueError):
        A.adamw_step(z, z, z, np.zeros(4), 1, 1e-3)


# ----------------------------------------------------- planted mistakes

def _planted(kind):
    def step(theta, g, m, v, t, lr, b1, b2, eps, wd):
        theta, g, m, v = (np.array(x, dtype=np.float64) for x in (theta, g, m, v))
        if kind == "l2_coupled":
            g = g + wd * theta
        if kind == "swapped_betas":
            b1, b2 = b2, b1
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m if kind == "no_bias_correction" else m / (1 - b1 ** t)
        vh = v if kind == "no_bias_correction" else v / (1 - b2 ** t)
        den = np.sqrt(vh + eps) if kind == "eps_inside_root" else np.sqrt(vh) + eps
        if kind == "l2_coupled":
            return theta - lr * mh / den, m, v
        if kind == "decay_after_update":
            return (1 - lr * wd) * (theta - lr * mh / den), m, v
        if kind == "no_decay":
            return theta - lr * mh / den, m, v
        return (1 - lr * wd) * theta - lr * mh / den, m, v
    return step


@pytest.mark.parametrize("kind", ["no_bias_correction", "eps_inside_root", "l2_coupled", "swapped_betas",
                                  "decay_after_update", "no_decay"])
def test_planted_adamw_mistakes_are_caught(kind):
    fn = _planted(kind)
    caught = 0
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught planted mistake {kind}"


def test_unplanted_reference_passes_every_pin():
    # the planting helper itself, with no mistake, passes: the pins test the mistakes, not the helper
    fn = _planted("none")
    for pin in PINS:
        pin(fn)
