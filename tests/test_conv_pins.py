"""Pins of the oracle's input-side convolution (oracle/conv.py).

Against an independent library routine (scipy.signal.lfilter: a causal FIR filter with
taps w[c][W-1-j], zero initial conditions), closed forms (W = 1, an impulse), SiLU's own
identities, and the speculative semantics (accept-all equals one-by-one decoding; a
rejected draft leaves no trace).
"""
import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

from oracle.conv import ConvOracle, silu


def _run_committed(oracle, xs, w, b, act):
    return np.concatenate([oracle.step(xs[:, t:t + 1], w, b, act, commit=True) for t in range(xs.shape[1])], axis=1)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_equals_a_causal_fir_filter(W):
    rng = np.random.default_rng(W)
    B, D, n = 2, 5, 12
    x = rng.standard_normal((B, n, D))
    w = rng.standard_normal((D, W))
    bias = rng.standard_normal(D)
    y = _run_committed(ConvOracle(B, D, W), x, w, bias, act=False)
    for bb in range(B):
        for c in range(D):
            # y_t = sum_j w[c][j] x_{t-W+1+j}: FIR taps h[m] = w[c][W-1-m]
            ref = lfilter(w[c, ::-1], [1.0], x[bb, :, c]) + bias[c]
            np.testing.assert_allclose(y[bb, :, c], ref, rtol=1e-12, atol=1e-12)


def test_width_one_is_pointwise_and_impulse_response():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 6, 3))
    w = rng.standard_normal((3, 1))
    b = rng.standard_normal(3)
    y = _run_committed(ConvOracle(1, 3, 1), x, w, b, act=True)
    np.testing.assert_allclose(y, silu(w[:, 0] * x + b), rtol=1e-14)
    # an impulse at t = 0 reads out the taps in reverse order of j
    W = 4
    imp = np.zeros((1, 6, 2))
    imp[0, 0] = 1.0
    w4 = rng.standard_normal((2, W))
    y4 = _run_committed(ConvOracle(1, 2, W), imp, w4, None, act=False)
    np.testing.assert_allclose(y4[0, :W], w4[:, ::-1].T, rtol=1e-15)
    np.testing.assert_array_equal(y4[0, W:], 0.0)


def test_silu_identities():
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(silu(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert silu(0.0) == 0.0
    # silu(z) - silu(-z) = z
    np.testing.assert_allclose(silu(z) - silu(-z), z, rtol=1e-12, atol=1e-12)


def test_speculative_rounds_match_committed_decoding():
    rng = np.random.default_rng(3)
    B, D, W, T = 3, 4, 4, 4
    w = rng.standard_normal((D, W))
    b = rng.standard_normal(D)
    spec, ref = ConvOracle(B, D, W), ConvOracle(B, D, W)
    for _ in range(6):
        x = rng.standard_normal((B, T, D))
        a = rng.integers(0, T + 1, size=B)
        y = spec.step(x, w, b)
        spec.accept(a)
        for bb in range(B):
            # a reference that sees only this sequence's accepted inputs, one at a time
            one = ConvOracle(1, D, W)
            one.history[0] = ref.history[bb].copy()
            yr = _run_committed(one, x[bb:bb + 1], w, b, act=True)
            np.testing.assert_allclose(y[bb], yr[0], rtol=1e-13)  # draft outputs as if committed
            ref.history[bb] = np.concatenate([ref.history[bb], x[bb, :a[bb]]], axis=0)
    for bb in range(B):
        np.testing.assert_array_equal(spec.history[bb], ref.history[bb])


def test_rejected_drafts_leave_no_trace():
    rng = np.random.default_rng(4)
    o = ConvOracle(2, 4, 3)
    w = rng.standard_normal((4, 3))
    x0 = rng.standard_normal((2, 1, 4))
    o.step(x0, w, commit=True)
    before = [h.copy() for h in o.history]
    o.step(rng.standard_normal((2, 4, 4)), w)
    o.accept(np.zeros(2, int))
    for bb in range(2):
        np.testing.assert_array_equal(o.history[bb], before[bb])
