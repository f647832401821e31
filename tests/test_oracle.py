"""Pins for the CPU oracle (runs on the CPU, no GPU).

The oracle is trusted only through these checks, each of which ties it to
something other than itself: brute-force sums on tiny inputs, closed forms,
hand-derived fixtures in tests/golden/, or an independent library routine
(numpy.fft, numpy.convolve, scipy.signal.lfilter).  Together they are chosen
so that a dropped term, a wrong sign, a wrong index or a swapped operand in
any oracle routine fails at least one of them (tests/test_oracle_mutants.py
plants such mistakes in a copy of the oracle and checks exactly that).
"""
import json
import os

import numpy as np
import pytest
import scipy.signal

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_dft(x, sign=-1):
    M = x.size
    n = np.arange(M)
    return np.array([np.sum(x * np.exp(sign * 2j * np.pi * f * n / M)) for f in range(M)])


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ----------------------------------------------------------------------- FFT
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 64, 256, 1024])
@pytest.mark.parametrize("sign", [-1, 1])
def test_fft_matches_bruteforce_dft(M, sign):
    rng = np.random.default_rng(M)
    x = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    assert _rel(oracle.fft(x, sign), brute_dft(x, sign)) < 1e-12


@pytest.mark.parametrize("M", [2 ** 12, 2 ** 16, 2 ** 18])
def test_fft_matches_numpy(M):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    assert _rel(oracle.fft(x, -1), np.fft.fft(x)) < 1e-12
    assert _rel(oracle.fft(x, +1), np.fft.ifft(x) * M) < 1e-12


@pytest.mark.parametrize("M", [8, 1024, 2 ** 20])
def test_fft_closed_forms(M):
    n = np.arange(M)
    delta = np.zeros(M, complex)
    delta[0] = 1
    assert np.allclose(oracle.fft(delta), np.ones(M), atol=1e-13)
    ones = np.ones(M, complex)
    X = oracle.fft(ones)
    assert abs(X[0] - M) < 1e-9 * M and np.max(np.abs(X[1:])) < 1e-9 * M
    f0 = M // 8 + 1 if M > 8 else 3
    e = np.exp(2j * np.pi * f0 * n / M)
    X = oracle.fft(e)
    assert abs(X[f0] - M) < 1e-8 * M
    X[f0] = 0
    assert np.max(np.abs(X)) < 1e-8 * M
    # shifted delta -> pure phase ramp
    d3 = np.zeros(M, complex)
    d3[3] = 1
    assert np.allclose(oracle.fft(d3), np.exp(-2j * np.pi * 3 * n / M), atol=1e-10)


def test_fft_parseval_hermitian_roundtrip():
    rng = np.random.default_rng(3)
    M = 4096
    x = rng.standard_normal(M)
    X = oracle.fft(x)
    assert abs(np.sum(np.abs(X) ** 2) / M - np.sum(x * x)) < 1e-10 * np.sum(x * x)
    assert np.allclose(X[1:], np.conj(X[1:][::-1]), atol=1e-10)
    z = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    assert _rel(oracle.fft(oracle.fft(z, -1), +1) / M, z) < 1e-13


def test_fft_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fft(np.ones(12))


# ------------------------------------------------------------ golden fixtures
def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["tiny_gated_conv.json", "tiny_ungated_partial.json"])
def test_hand_derived_golden(name):
    g = _load_golden(name)
    u = np.array(g["u"], float)[None, None]
    k = np.array(g["k"], float)[None]
    w = None if g["w"] is None else np.array(g["w"], float)[None, None]
    v = None if g["v"] is None else np.array(g["v"], float)[None, None]
    want = np.array(g["y"], float)
    assert np.array_equal(oracle.direct(u, k, w, v)[0, 0], want)
    assert np.max(np.abs(oracle.fft_conv(u, k, w, v)[0, 0] - want)) < 1e-12


def test_golden_dc_only_mask():
    g = _load_golden("dc_only_mask.json")
    N = g["N"]
    rng = np.random.default_rng(g["seed"])
    u = rng.standard_normal((1, 1, N))
    k = rng.standard_normal((1, N))
    mask = np.zeros((1, 128), np.uint8)
    mask[0, 0] = 1      # with N = 128 each block is one bin: only the DC bin survives
    y = oracle.fft_conv(u, k, mask=mask)[0, 0]
    want = np.full(N, k.sum() * u.sum() / (2 * N))
    assert np.max(np.abs(y - want)) < 1e-12 * max(1.0, np.abs(want).max())


# -------------------------------------------------------------- convolution
def _inputs(B, H, N, L, gated, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, H, N))
    k = rng.standard_normal((H, L)) * np.exp(-0.05 * np.arange(L))
    w = rng.standard_normal((B, H, N)) if gated else None
    v = rng.standard_normal((B, H, N)) if gated else None
    return u, k, w, v


@pytest.mark.parametrize("B,H,N,L,gated", [(1, 1, 16, 16, False), (2, 3, 64, 17, True),
                                           (3, 2, 128, 1, True), (1, 4, 256, 256, True)])
def test_direct_matches_numpy_convolve(B, H, N, L, gated):
    u, k, w, v = _inputs(B, H, N, L, gated, 11)
    y = oracle.direct(u, k, w, v)
    for b in range(B):
        for h in range(H):
            x = u[b, h] * (w[b, h] if gated else 1.0)
            ref = np.convolve(x, k[h])[:N] * (v[b, h] if gated else 1.0)
            assert _rel(y[b, h], ref) < 1e-13


@pytest.mark.parametrize("B,H,N,L,gated", [(1, 1, 16, 16, False), (2, 3, 64, 17, True),
                                           (3, 2, 128, 1, True), (1, 4, 1024, 1024, False),
                                           (2, 2, 512, 300, True)])
def test_fft_route_matches_direct(B, H, N, L, gated):
    u, k, w, v = _inputs(B, H, N, L, gated, 12)
    yd = oracle.direct(u, k, w, v)
    yf, imag = oracle.fft_conv(u, k, w, v, return_imag=True)
    assert _rel(yf, yd) < 1e-12
    assert imag < 1e-12


def test_direct_points_match_direct():
    u, k, w, v = _inputs(2, 3, 200, 50, True, 13)
    y = oracle.direct(u, k, w, v)
    rng = np.random.default_rng(0)
    pts = np.stack([rng.integers(0, 2, 40), rng.integers(0, 3, 40), rng.integers(0, 200, 40)], 1)
    yp = oracle.direct_points(u, k, pts, w, v)
    assert np.array_equal(yp, y[pts[:, 0], pts[:, 1], pts[:, 2]])


def test_delta_filters():
    u, _, w, v = _inputs(2, 2, 128, 1, True, 14)
    k0 = np.zeros((2, 128))
    k0[:, 0] = 1.0
    assert np.array_equal(oracle.direct(u, k0, w, v), v * (u * w))
    assert np.max(np.abs(oracle.fft_conv(u, k0, w, v) - v * (u * w))) < 1e-13
    d = 5
    kd = np.zeros((2, 128))
    kd[:, d] = 1.0
    want = np.zeros_like(u)
    want[..., d:] = (u * w)[..., :-d]
    want *= v
    assert np.array_equal(oracle.direct(u, kd, w, v), want)
    assert np.max(np.abs(oracle.fft_conv(u, kd, w, v) - want)) < 1e-13


@pytest.mark.parametrize("N,L,a", [(1 << 12, 1 << 12, 0.999), (1 << 16, 1 << 15, 0.9999),
                                   (1 << 20, 1 << 20, 0.99999)])
def test_exponential_filter_is_iir(N, L, a):
    """k[t] = a^t, t < L  <=>  y[t] = a y[t-1] + x[t] - a^L x[t-L]  (closed form)."""
    rng = np.random.default_rng(N)
    x = rng.standard_normal(N)
    k = a ** np.arange(L, dtype=np.float64)
    xd = x.copy()
    xd[L:] -= a ** L * x[:-L] if L < N else 0.0
    ref = scipy.signal.lfilter([1.0], [1.0, -a], xd)   # first-order recursion, O(N)
    y = oracle.fft_conv(x[None, None], k[None])[0, 0]
    assert _rel(y, ref) < 1e-10


def test_integer_prefix_sums_are_exact():
    """All-ones filter of length L on integer input = windowed sums, exact in float64."""
    rng = np.random.default_rng(5)
    N, L = 4096, 1000
    x = rng.integers(-8, 9, N).astype(float)
    c = np.concatenate([[0.0], np.cumsum(x)])
    t = np.arange(N)
    ref = c[t + 1] - c[np.maximum(t + 1 - L, 0)]
    y = oracle.fft_conv(x[None, None], np.ones((1, L)))[0, 0]
    assert np.array_equal(np.round(y), ref)
    assert np.max(np.abs(y - ref)) < 1e-7
    assert np.array_equal(oracle.direct(x[None, None], np.ones((1, L)))[0, 0], ref)


def test_zero_padding_independence():
    u, k, w, v = _inputs(1, 2, 256, 256, True, 15)
    assert _rel(oracle.fft_conv(u, k, w, v, M=512), oracle.fft_conv(u, k, w, v, M=2048)) < 1e-13


def test_causality():
    u, k, w, v = _inputs(1, 1, 512, 512, True, 16)
    t0 = 300
    u2 = u.copy()
    u2[..., t0] += 10.0
    yd, yd2 = oracle.direct(u, k, w, v), oracle.direct(u2, k, w, v)
    assert np.array_equal(yd[..., :t0], yd2[..., :t0])
    assert not np.allclose(yd[..., t0:], yd2[..., t0:])
    yf, yf2 = oracle.fft_conv(u, k, w, v), oracle.fft_conv(u2, k, w, v)
    assert np.max(np.abs(yf[..., :t0] - yf2[..., :t0])) < 1e-12 * np.abs(yf).max()


def test_linearity_and_unit_gates():
    u, k, w, v = _inputs(2, 2, 256, 100, True, 17)
    u2, k2, _, _ = _inputs(2, 2, 256, 100, False, 18)
    y = oracle.fft_conv(2.0 * u + u2, k, None, None)
    assert _rel(y, 2.0 * oracle.fft_conv(u, k) + oracle.fft_conv(u2, k)) < 1e-13
    y = oracle.fft_conv(u, 3.0 * k - k2)
    assert _rel(y, 3.0 * oracle.fft_conv(u, k) - oracle.fft_conv(u, k2)) < 1e-13
    ones = np.ones_like(u)
    assert _rel(oracle.fft_conv(u, k, ones, ones), oracle.fft_conv(u, k)) < 1e-15
    # w gates the input, v the output: the two are not interchangeable
    assert not np.allclose(oracle.direct(u, k, w, v), oracle.direct(u, k, v, w))


def test_partial_filter_equals_zero_appended():
    u, k, w, v = _inputs(1, 3, 512, 37, True, 19)
    kz = np.zeros((3, 512))
    kz[:, :37] = k
    assert _rel(oracle.fft_conv(u, k, w, v), oracle.fft_conv(u, kz, w, v)) < 1e-13
    assert np.array_equal(oracle.direct(u, k, w, v), oracle.direct(u, kz, w, v))


# ---------------------------------------------------------------------- mask
def _numpy_masked_reference(u, k, w, v, mask):
    """Independent route: numpy rfft/irfft with masked bins, then a direct circular sum."""
    B, H, N = u.shape
    M = 2 * N
    G = N // 128
    out = np.zeros_like(u)
    for h in range(H):
        K = np.fft.rfft(np.concatenate([k[h], np.zeros(M - k.shape[1])]))
        blk = np.minimum(np.arange(N + 1) // G, 127)
        K = K * mask[h, blk]
        kp = np.fft.irfft(K, n=M)
        for b in range(B):
            x = np.concatenate([u[b, h] * (w[b, h] if w is not None else 1.0), np.zeros(N)])
            idx = (np.arange(N)[:, None] - np.arange(M)[None, :]) % M
            c = (kp[None, :] * x[idx]).sum(axis=1)
            out[b, h] = c * (v[b, h] if v is not None else 1.0)
    return out


def test_mask_all_ones_equals_dense_and_all_zero_is_zero():
    u, k, w, v = _inputs(2, 3, 256, 256, True, 20)
    ones = np.ones((3, 128), np.uint8)
    assert _rel(oracle.fft_conv(u, k, w, v, mask=ones), oracle.fft_conv(u, k, w, v)) < 1e-15
    zeros = np.zeros((3, 128), np.uint8)
    assert np.max(np.abs(oracle.fft_conv(u, k, w, v, mask=zeros))) < 1e-14


@pytest.mark.parametrize("kind", ["band", "random"])
def test_mask_matches_numpy_circular(kind):
    N = 256
    u, k, w, v = _inputs(2, 2, N, 200, True, 21)
    if kind == "band":
        mask = np.zeros((2, 128), np.uint8)
        mask[:, :27] = 1
    else:
        mask = (np.random.default_rng(3).random((2, 128)) < 0.5).astype(np.uint8)
    y = oracle.fft_conv(u, k, w, v, mask=mask)
    ref = _numpy_masked_reference(u, k, w, v, mask)
    assert _rel(y, ref) < 1e-12
    # the circular-form sampled route agrees too
    kp = oracle.masked_filter(k[1], N, mask[1])
    ts = np.array([0, 1, 77, 255])
    yp = oracle.circular_points(u[1, 1], kp, ts, w[1, 1], v[1, 1])
    assert np.max(np.abs(yp - ref[1, 1, ts])) < 1e-12 * np.abs(ref).max()


def test_mask_is_idempotent_on_the_filter():
    """Applying the masked filter's own spectrum mask again changes nothing."""
    N = 512
    rng = np.random.default_rng(22)
    k = rng.standard_normal(N)
    mask = np.zeros(128, np.uint8)
    mask[:40] = 1
    kp = oracle.masked_filter(k, N, mask)
    # kp is a length-2N circular filter; re-masking its own spectrum is a no-op
    K = np.fft.fft(kp)
    f = np.arange(2 * N)
    fr = np.where(f <= N, f, 2 * N - f)
    assert np.max(np.abs(K[mask[np.minimum(fr // (N // 128), 127)] == 0])) < 1e-12
