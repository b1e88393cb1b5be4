"""Pins for the oracle's Euler and bilinear discretization rules
("State-space models", section "Discretization"; "Structured State Space
Models and Mamba ...", section "Discretization Mechanics: Zero-Order Hold and
Bilinear Transforms").

- the page's statements for a = -1 (tests/golden/discretization_rules.txt),
  read off the scan's impulse response;
- each rule as the step of a numerical integrator of dh/dt = a h + b u:
  forward Euler h_t = h_{t-1} + delta (a h_{t-1} + b u_t), and the trapezoidal
  rule h_t (1 - delta a / 2) = h_{t-1} (1 + delta a / 2) + delta b u_t;
- the LTI kernel by powers equals the kernel by repeated products, and equals
  the recurrence's impulse response, under every rule;
- all rules agree to first order as the step goes to zero."""
import numpy as np
import pytest

import oracle
from conftest import load_golden

RULES = ("delta", "zoh", "euler", "bilinear")


def _scalar_scan(a, dts, u, b=1.0, c=1.0, rule="euler", h0=None):
    L = len(u)
    y, fs = oracle.selective_scan(
        np.asarray(u, dtype=np.float64).reshape(1, 1, L),
        np.asarray(dts, dtype=np.float64).reshape(1, 1, L), np.array([[a]]),
        np.full((1, 1, L), b), np.full((1, 1, L), c), delta_softplus=False, bbar=rule,
        h0=None if h0 is None else np.array([[h0]]))
    return y.reshape(L), fs.reshape(1)


def _abar(a, dt, rule):
    y, _ = _scalar_scan(a, [dt, dt], [1.0, 0.0], rule=rule)
    return y[1] / y[0]


def test_page_statements_for_a_minus_one():
    g = load_golden("discretization_rules.txt")
    a = g["a"][0]
    for dt, want in g["euler_abar"]:
        assert abs(_abar(a, dt, "euler") - want) < 1e-12
    thr = g["euler_unstable_above"][0]
    for dt in np.linspace(0.05, 4.0, 80):
        assert (abs(_abar(a, dt, "euler")) > 1.0) == (dt > thr + 1e-12), dt
    assert abs(_abar(a, g["bilinear_stable_at"][0], "bilinear")) < 1.0
    dt = g["closer_at"][0]
    exact = np.exp(a * dt)
    assert abs(_abar(a, dt, "bilinear") - exact) < abs(_abar(a, dt, "euler") - exact)


def test_bilinear_stable_for_every_step():
    for a in (-0.01, -1.0, -16.0):
        for dt in np.geomspace(1e-4, 1e4, 41):
            assert abs(_abar(a, dt, "bilinear")) < 1.0


@pytest.mark.parametrize("rule", ["euler", "bilinear"])
def test_rules_are_integrator_steps(rule):
    r = np.random.default_rng(5)
    L = 40
    a, b = -0.7, 1.3
    dts = r.uniform(0.01, 1.5, L)
    u = r.standard_normal(L)
    h, _ = _scalar_scan(a, dts, u, b=b, c=1.0, rule=rule, h0=0.4)  # y_t = h_t
    prev = np.concatenate([[0.4], h[:-1]])
    if rule == "euler":
        want = prev + dts * (a * prev + b * u)
        assert np.allclose(h, want, rtol=1e-13, atol=1e-13)
    else:
        lhs = h * (1 - dts * a / 2)
        rhs = prev * (1 + dts * a / 2) + dts * b * u
        assert np.allclose(lhs, rhs, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rule", RULES)
def test_lti_kernel_powers_products_and_impulse_response(rule):
    r = np.random.default_rng(9)
    D, N, L = 3, 4, 24
    A = -r.uniform(0.1, 2.0, (D, N))
    Bv, Cv = r.standard_normal((D, N)), r.standard_normal((D, N))
    delta = np.array([0.3, 1.0, 2.5])  # Euler at 1.0 and 2.5 gives Abar = 0 and negative values
    K0 = oracle.lti_kernel(A, Bv, Cv, delta, L, bbar=rule, method="direct")
    K1 = oracle.lti_kernel(A, Bv, Cv, delta, L, bbar=rule, method="powers")
    assert np.allclose(K0, K1, rtol=1e-12, atol=1e-12)
    # impulse response of the recurrence with the same constant step and B, C
    for d in range(D):
        u = np.zeros((1, 1, L))
        u[0, 0, 0] = 1.0
        y, _ = oracle.selective_scan(u, np.full((1, 1, L), delta[d]), A[d:d + 1],
                                     np.repeat(Bv[d][None, :, None], L, axis=2),
                                     np.repeat(Cv[d][None, :, None], L, axis=2), bbar=rule)
        assert np.allclose(y.reshape(L), K0[d], rtol=1e-12, atol=1e-12)


def test_rules_agree_to_first_order():
    a = -1.7
    for dt in (1e-2, 1e-3):
        vals = [_abar(a, dt, rule) for rule in RULES]
        assert max(vals) - min(vals) < 2 * (a * dt) ** 2
