"""Pins of the oracle's decay-from-time-step function (oracle/decay.py).

Each pin is fixed by the mathematics, not by retyping the formula: softplus(0) =
ln 2, the limits of softplus, its reflection identity softplus(x) - softplus(-x)
= x, and softplus as the integral of the logistic function.
"""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle.decay import alpha_from_dt, softplus


def test_zero_time_step_gives_a_power_of_two():
    # softplus(0) = ln 2, so alpha = exp(-A ln 2) = 2^-A
    A = np.array([0.5, 1.0, 2.0, 3.0])
    np.testing.assert_allclose(alpha_from_dt(np.zeros(4), A), 2.0 ** -A, rtol=1e-15)


def test_bias_shifts_the_time_step():
    A = np.array([1.5, 0.7])
    dt = np.array([[0.3, -1.2], [2.0, 0.0]])
    b = np.array([-0.3, 1.2])
    np.testing.assert_allclose(alpha_from_dt(dt, A, b), alpha_from_dt(dt + b, A), rtol=1e-15)
    np.testing.assert_array_equal(alpha_from_dt(dt, A, None), alpha_from_dt(dt, A, np.zeros(2)))
    # bias -dt: a zero time step
    np.testing.assert_allclose(alpha_from_dt(np.array([[0.3, -1.2]]), A, np.array([-0.3, 1.2]))[0], 2.0 ** -A,
                               rtol=1e-15)


def test_limits():
    # a very negative time step: no decay; A = 0: no decay
    assert alpha_from_dt(np.array([-800.0]), np.array([2.0]))[0] == 1.0
    assert alpha_from_dt(np.array([5.0]), np.array([0.0]))[0] == 1.0
    # a large time step: softplus(x) = x + log1p(e^-x), so alpha ~ exp(-x A)
    x, A = 30.0, 0.5
    np.testing.assert_allclose(alpha_from_dt(np.array([x]), np.array([A]))[0], math.exp(-x * A), rtol=1e-12)


@pytest.mark.parametrize("x", [-6.0, -1.5, -0.25, 0.1, 0.8, 3.0, 9.0])
def test_reflection_identity(x):
    # softplus(x) - softplus(-x) = x, hence alpha(x) / alpha(-x) = exp(-x A): a sign slip fails it
    A = 1.3
    r = alpha_from_dt(np.array([x]), np.array([A]))[0] / alpha_from_dt(np.array([-x]), np.array([A]))[0]
    np.testing.assert_allclose(r, math.exp(-x * A), rtol=1e-13)


@pytest.mark.parametrize("x", [-4.0, -0.5, 0.0, 1.0, 2.5, 6.0])
def test_softplus_is_the_integral_of_the_logistic(x):
    val, err = integrate.quad(lambda t: 1.0 / (1.0 + math.exp(-t)), -60.0, x, epsabs=1e-14, epsrel=1e-13)
    np.testing.assert_allclose(softplus(x), val, rtol=1e-11, atol=1e-14)


def test_decay_is_in_unit_interval_and_decreasing():
    dt = np.linspace(-10, 10, 201)
    a = alpha_from_dt(dt, np.full_like(dt, 1.7))
    assert np.all(a > 0) and np.all(a <= 1) and np.all(np.diff(a) < 0)
