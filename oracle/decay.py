"""The decay of a record from its raw time step, in fp64 -- TEST INFRASTRUCTURE ONLY.

Mamba-2's discretisation of the layer just before the decode path (the step that
produces the alpha the records carry; "ReplaySSM: Cache SSM Inputs, Not State",
How it works: the buffer holds (alpha, k, v) per token):

    Delta = softplus(dt + dt_bias),  alpha = exp(-Delta * A)

with softplus(x) = log(1 + e^x) per (sequence, token, head) and A, dt_bias per
head. Written as the plain definition, with numpy's logaddexp(0, x) = log(e^0 + e^x)
as the one library step.
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x), elementwise, in fp64."""
    return np.logaddexp(0.0, np.asarray(x, np.float64))


def alpha_from_dt(dt, A, dt_bias=None):
    """dt [..., H] (any leading axes), A [H], dt_bias [H] or None -> alpha [..., H] in fp64."""
    x = np.asarray(dt, np.float64)
    if dt_bias is not None:
        x = x + np.asarray(dt_bias, np.float64)
    return np.exp(-softplus(x) * np.asarray(A, np.float64))
