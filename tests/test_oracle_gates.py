"""Pins of the oracle's gate activations (oracle/gates.py) to closed forms:
sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, softplus(0) = ln 2, softplus(ln(e - 1)) = 1,
the lower bound, and the head of each column (c // D for KDA, c for GDN)."""
import math

import numpy as np

from oracle import gates


def test_sigmoid_form_closed_values():
    D, lb = 2, -5.0
    A_log = np.array([0.0, math.log(2.0)])  # e^A = 1 and 2
    bias = np.zeros(4)
    x0 = np.zeros((1, 1, 4))
    np.testing.assert_allclose(gates.gate_sigmoid(x0, A_log, bias, lb, D), -2.5, rtol=0, atol=1e-15)
    # e^A (x + bias) = ln 3 in every column -> sigmoid = 3/4
    x = np.array([[[math.log(3.0)] * 2 + [math.log(3.0) / 2] * 2]])
    np.testing.assert_allclose(gates.gate_sigmoid(x, A_log, bias, lb, D), -3.75, rtol=1e-15)
    # the bias is added before the head factor: x = 0, bias = ln 3 on head 0
    g = gates.gate_sigmoid(x0, A_log, np.array([math.log(3.0)] * 2 + [0.0] * 2), lb, D)
    np.testing.assert_allclose(g[0, 0], [-3.75, -3.75, -2.5, -2.5], rtol=1e-15)


def test_softplus_form_closed_values_and_bound():
    D = 2
    a = np.array([-1.0, -2.0])
    bias = np.zeros(4)
    g = gates.gate_softplus(np.zeros((1, 1, 4)), a, bias, -math.inf, D)
    np.testing.assert_allclose(g[0, 0], [-math.log(2)] * 2 + [-2 * math.log(2)] * 2, rtol=1e-15)
    g = gates.gate_softplus(np.full((1, 1, 4), math.log(math.e - 1.0)), a, bias, -math.inf, D)
    np.testing.assert_allclose(g[0, 0], [-1.0, -1.0, -2.0, -2.0], rtol=1e-14)
    # softplus(10) = 10 + ln(1 + e^-10): head 0 gives -10.0000454 (above a bound of -15),
    # head 1 gives -20.0000908 (clamped there)
    sp10 = 10.0 + math.log1p(math.exp(-10.0))
    g = gates.gate_softplus(np.full((1, 1, 4), 10.0), a, bias, -15.0, D)
    np.testing.assert_allclose(g[0, 0], [-sp10, -sp10, -15.0, -15.0], rtol=1e-14)


def test_gdn_columns_are_heads():
    a = np.array([-1.0, -3.0, -0.5])
    g = gates.gate_softplus(np.zeros((2, 5, 3)), a, np.zeros(3), -math.inf, D=128, gdn=True)
    np.testing.assert_allclose(g[1, 4], a * math.log(2.0), rtol=1e-15)
    g = gates.gate_sigmoid(np.zeros((1, 1, 3)), np.zeros(3), np.zeros(3), -4.0, D=128, gdn=True)
    np.testing.assert_allclose(g, -2.0, rtol=1e-15)


def test_beta_sigmoid():
    np.testing.assert_allclose(gates.beta_sigmoid([0.0, math.log(3.0), -math.log(3.0)]), [0.5, 0.75, 0.25],
                               rtol=1e-15)
