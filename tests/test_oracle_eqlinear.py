"""Pins of the group-axis circular-convolution oracle (Flash EQ-Linear
abstract page: circular convolution along the group dimension composed with
a channel linear map), each independent of the oracle's own loop."""
import numpy as np
import pytest

from oracle.eqlinear import eqlinear, eqlinear_tokens


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_equals_block_circulant_dense_layer():
    # the unrolled dense layer: block (t, t') of the (T C_out) x (T C_in) matrix is W[(t - t') mod T]
    N, T, Ci, Co = 5, 6, 3, 4          # C_out != C_in catches a transposed W
    x, W = _rand(1, N, T, Ci), _rand(2, T, Co, Ci)
    M = np.zeros((T * Co, T * Ci))
    for t in range(T):
        for tp in range(T):
            M[t * Co:(t + 1) * Co, tp * Ci:(tp + 1) * Ci] = W[(t - tp) % T]
    dense = (x.reshape(N, T * Ci) @ M.T).reshape(N, T, Co)
    np.testing.assert_allclose(eqlinear(x, W), dense, rtol=1e-12, atol=1e-12)


def test_identity_and_shift_closed_forms():
    N, T, C = 4, 8, 5
    x = _rand(3, N, T, C)
    W = np.zeros((T, C, C))
    W[0] = np.eye(C)
    np.testing.assert_allclose(eqlinear(x, W), x, atol=1e-15)
    for s0 in (1, 3, 7):
        W = np.zeros((T, C, C))
        W[s0] = np.eye(C)
        y = eqlinear(x, W)
        for t in range(T):
            np.testing.assert_allclose(y[:, t], x[:, (t - s0) % T], atol=1e-15)


def test_equivariance_under_group_shifts():
    N, T, Ci, Co = 3, 8, 4, 6
    x, W = _rand(4, N, T, Ci), _rand(5, T, Co, Ci)
    y = eqlinear(x, W)
    for r in (1, 2, 5):
        np.testing.assert_allclose(eqlinear(np.roll(x, r, axis=1), W), np.roll(y, r, axis=1),
                                   rtol=1e-12, atol=1e-12)


def test_single_channel_is_fft_circular_convolution():
    N, T = 7, 16
    x, W = _rand(6, N, T, 1), _rand(7, T, 1, 1)
    ref = np.real(np.fft.ifft(np.fft.fft(x[:, :, 0], axis=1) * np.fft.fft(W[:, 0, 0])[None, :], axis=1))
    np.testing.assert_allclose(eqlinear(x, W)[:, :, 0], ref, rtol=1e-10, atol=1e-12)


def test_fourier_route_per_frequency_matrix():
    # real DFT along the group axis; per frequency the channel map is a complex matrix
    N, T, Ci, Co = 4, 8, 3, 2
    x, W = _rand(8, N, T, Ci), _rand(9, T, Co, Ci)
    X = np.fft.rfft(x, axis=1)                     # (N, T/2+1, Ci)
    Wf = np.fft.rfft(W, axis=0)                    # (T/2+1, Co, Ci)
    Y = np.einsum("fdc,nfc->nfd", Wf, X)
    ref = np.fft.irfft(Y, n=T, axis=1)
    np.testing.assert_allclose(eqlinear(x, W), ref, rtol=1e-10, atol=1e-12)


def test_token_subset_and_shapes():
    x, W = _rand(10, 9, 4, 2), _rand(11, 4, 3, 2)
    np.testing.assert_allclose(eqlinear_tokens(x, W, [0, 4, 8]), eqlinear(x, W)[[0, 4, 8]])
    with pytest.raises(ValueError):
        eqlinear(x, W[:, :, :1])
