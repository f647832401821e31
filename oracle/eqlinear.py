"""CPU oracle for the group-axis circular convolution (float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
package smoke check and the benchmark's CPU-baseline leg are its only users,
and the HIP library never calls it.

What is computed (the Flash EQ-Linear abstract page: the equivariant linear
layer is a circular convolution along the group dimension composed with a
linear map along the channel dimension).  With x (N, T, C_in) -- N tokens, a
cyclic group of order T, C_in channels -- and one channel matrix per group
offset, W (T, C_out, C_in):

    y[n, t, d] = sum_{s < T} sum_{c < C_in} W[s, d, c] * x[n, (t - s) mod T, c]

The plain definition is written out below, one group offset at a time; it is
pinned in the tests to the unrolled block-circulant dense layer the page
contrasts with, to closed forms (identity, shifts), to the equivariance
property and, for one channel, to numpy's FFT circular convolution.
"""
from __future__ import annotations

import numpy as np


def eqlinear(x, W) -> np.ndarray:
    """y (N, T, C_out) = sum_s x rolled by s along the group axis, times W[s]^T."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    N, T, C_in = x.shape
    Ts, C_out, C_in2 = W.shape
    if Ts != T or C_in2 != C_in:
        raise ValueError("shape mismatch: x (N, T, C_in), W (T, C_out, C_in)")
    y = np.zeros((N, T, C_out), dtype=np.float64)
    for s in range(T):
        # shifted[:, t, :] = x[:, (t - s) mod T, :]
        shifted = np.roll(x, s, axis=1)
        y += shifted @ W[s].T
    return y


def eqlinear_tokens(x, W, tokens) -> np.ndarray:
    """The definition at selected token rows only: y[tokens] (len(tokens), T, C_out)."""
    x = np.asarray(x)[np.asarray(tokens)]
    return eqlinear(x, W)
