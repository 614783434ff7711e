"""Pins of the oracle's in-kernel prologue (oracle/prologue.py) to closed forms.

The prologue: -exp(A_log) softplus(x + dt_bias) or lower_bound sigmoid(exp(A_log)(x + dt_bias)) for
the gate (KDA source walk-through, section 2), sigma(beta) and the L2 norm of q and k rows (FlashKDA
section of the same page).  Each piece is checked at points whose value is known exactly, and the
pieces are checked to invert: raw inputs built from target values by the inverse functions come
back as those targets."""
import math

import numpy as np
import pytest

from oracle.prologue import L2_EPS, apply_prologue, gate_activation, l2norm_rows, sigmoid, softplus
from oracle.recurrent import gdn_recurrent


def test_softplus_closed_forms():
    assert softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert softplus(40.0) == pytest.approx(40.0, rel=1e-15)
    assert softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)   # log(1 + e^-40) = e^-40 (1 - ...)
    assert softplus(math.log(3.0)) == pytest.approx(math.log(4.0), rel=1e-15)


def test_sigmoid_closed_forms():
    assert sigmoid(0.0) == 0.5
    assert sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    x = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(sigmoid(x) + sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert sigmoid(-800.0) == 0.0 and sigmoid(800.0) == 1.0   # no overflow warnings in either tail


def test_gate_activation_softplus_form():
    # x + dt_bias = 0: softplus = ln 2, so g = -exp(A_log) ln 2
    A_log = np.log(np.array([0.5, 2.0]))
    g = gate_activation(np.array([[0.3, -1.0]]), A_log, dt_bias=np.array([-0.3, 1.0]))
    np.testing.assert_allclose(g, [[-0.5 * math.log(2.0), -2.0 * math.log(2.0)]], rtol=1e-15)
    # x + dt_bias = ln 3: softplus = ln 4
    g = gate_activation(np.array([math.log(3.0)]), np.array([0.0]))
    assert g[0] == pytest.approx(-math.log(4.0), rel=1e-15)


def test_gate_activation_lower_bound_form():
    A_log = np.array([math.log(2.0)])
    assert gate_activation(np.array([0.0]), A_log, lower_bound=-5.0)[0] == -2.5       # sigma(0) = 1/2
    assert gate_activation(np.array([50.0]), A_log, lower_bound=-5.0)[0] == pytest.approx(-5.0, rel=1e-15)
    assert gate_activation(np.array([-50.0]), A_log, lower_bound=-5.0)[0] == pytest.approx(0.0, abs=1e-40)
    # exp(A_log) (x + b) = ln 3: sigma = 3/4
    x = math.log(3.0) / 2.0
    assert gate_activation(np.array([x]), A_log, lower_bound=-4.0)[0] == pytest.approx(-3.0, rel=1e-15)


def test_gate_activation_per_channel_broadcast():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 2, 4))          # [T, H, D]
    A_log, b = rng.standard_normal(2), rng.standard_normal((2, 4))
    g = gate_activation(x, A_log, b, gate="channel")
    for t, h, d in [(0, 0, 0), (2, 1, 3), (1, 0, 2)]:
        want = -math.exp(A_log[h]) * math.log1p(math.exp(x[t, h, d] + b[h, d]))
        assert g[t, h, d] == pytest.approx(want, rel=1e-14)


def test_l2norm_rows():
    np.testing.assert_allclose(l2norm_rows(np.array([[3.0, 4.0]])), [[3 / math.sqrt(25 + L2_EPS), 4 / math.sqrt(25 + L2_EPS)]],
                               rtol=1e-15)
    np.testing.assert_array_equal(l2norm_rows(np.zeros((2, 8))), 0.0)          # no division by zero
    x = np.random.default_rng(1).standard_normal((5, 3, 64)) * 7.0
    n = np.linalg.norm(l2norm_rows(x), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=0, atol=1e-7)                         # eps / |x|^2 ~ 1e-9


def test_prologue_inverts_to_processed_inputs():
    # raw inputs made from processed targets by the inverse functions: the prologue returns the
    # targets, and the recurrence on them equals the recurrence on the targets
    rng = np.random.default_rng(2)
    T, H, D = 37, 2, 16
    q0 = l2norm_rows(rng.standard_normal((T, H, D)))
    k0 = l2norm_rows(rng.standard_normal((T, H, D)))
    v = rng.standard_normal((T, H, D))
    g0 = -rng.uniform(0.01, 0.5, (T, H))                 # target log-gates
    b0 = rng.uniform(0.05, 0.95, (T, H))                 # target betas
    A_log, dt = np.log(np.array([0.3, 0.8])), np.array([0.2, -0.1])
    # softplus^-1(y) = log(expm1(y)), sigmoid^-1(p) = log(p / (1 - p)); rows rescaled by positive factors
    x = np.log(np.expm1(-g0 / np.exp(A_log))) - dt
    bl = np.log(b0 / (1 - b0))
    c = np.exp(0.3 * rng.standard_normal((T, H, 1)))   # factors in ~[0.4, 2.5]: eps / |x|^2 <= 1e-5
    q, k, g, b = apply_prologue(c * q0, 2.0 * c * k0, x, bl, "scalar", True, True, A_log, dt)
    np.testing.assert_allclose(g, g0, rtol=1e-12)
    np.testing.assert_allclose(b, b0, rtol=1e-12)
    np.testing.assert_allclose(q, q0, rtol=1e-5)         # eps changes the scale by ~eps / |x|^2
    np.testing.assert_allclose(k, k0, rtol=1e-5)
    o1, s1 = gdn_recurrent(q, k, v, g, b, 0.25)
    o0, s0 = gdn_recurrent(q0, k0, v, g0, b0, 0.25)
    np.testing.assert_allclose(o1, o0, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(s1, s0, rtol=1e-4, atol=1e-6)
