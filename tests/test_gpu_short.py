"""GPU parity of the chunked short-filter path (fftconv_prepare_short_filter +
fftconv_fwd_short: overlap-save windows of 2048 samples at a hop of 1024, each a
2048-point circular convolution on the matrix cores) against the CPU oracle's
exact causal convolution with the same filter.

The second half of a window's circular convolution is free of wrap-around when
the filter has at most 1024 taps, so the result is the full causal convolution;
the cases cover the first window (zeros before the sequence), the longest filter,
an odd number of windows (the last window pair has one window), sequence lengths
that are multiples of 1024 but not powers of two, both gates, several channels
and batch rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import long_fft_convolution_amd as fc
from long_fft_convolution_amd import synth
from parity import check

pytestmark = pytest.mark.gpu

TOL = {"f16": 5e-3, "bf16": 2e-2}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(t):
    return None if t is None else t.cuda()


def _run(inp):
    y = fc.causal_conv_short(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v))
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _ref(inp):
    # direct O(N L) sums (any N); the radix-2 FFT route for long power-of-two N
    w = None if inp.w is None else inp.f64("w")
    v = None if inp.v is None else inp.f64("v")
    N = inp.u.shape[-1]
    if N & (N - 1) == 0 and N > 16384:
        return oracle.fft_conv(inp.f64("u"), inp.f64("k"), w, v)
    return oracle.direct(inp.f64("u"), inp.f64("k"), w, v)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,L", [(1024, 512), (1024, 1024), (2048, 1), (3072, 100), (3072, 1024),
                                 (8192, 511), (8192, 1023), (5 * 1024, 257), (7 * 1024, 1000)])
def test_short_filter_sizes(dtype, N, L):
    _say(f"short {dtype} N={N} L={L}")
    inp = synth.generate(3, 2, N, L, dtype, gated=True, seed=N + L)
    check(_run(inp), _ref(inp), TOL[dtype])


@pytest.mark.parametrize("gated", [False, True])
def test_short_filter_gates_and_batch(gated):
    N, L = 1 << 14, 300
    _say(f"short gated={gated} B=5 H=3 N={N}")
    inp = synth.generate(5, 3, N, L, "f16", gated=gated, seed=7)
    y = _run(inp)
    ref = _ref(inp)
    check(y, ref, TOL["f16"])
    # every window boundary is exact: the error is flat along the sequence
    err = np.abs(y - ref).reshape(5, 3, N // 1024, 1024).max(axis=(0, 1, 3))
    scale = np.abs(ref).max()
    assert err.max() < 2e-2 * scale


def test_short_filter_long_sequence():
    N, L = 1 << 20, 1024
    _say(f"short N={N} L={L} H=2")
    inp = synth.generate(1, 2, N, L, "f16", gated=False, seed=21)
    check(_run(inp), _ref(inp), TOL["f16"])


def test_short_filter_matches_full_path():
    # the same convolution through the full-length spectrum
    N, L = 1 << 15, 512
    _say(f"short vs full N={N}")
    inp = synth.generate(2, 2, N, L, "f16", gated=True, seed=5)
    y_short = _run(inp)
    y_full = fc.causal_conv(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v)).float().cpu().double().numpy()
    ref = _ref(inp)
    check(y_short, ref, TOL["f16"])
    check(y_full, ref, TOL["f16"])
    check(y_short, y_full, 2 * TOL["f16"])


def test_short_filter_empty_batch():
    u = torch.empty((0, 3, 2048), dtype=torch.float16, device="cuda")
    k = torch.randn(3, 64).to(torch.float16).cuda()
    out = fc.causal_conv_short(u, k)
    assert out.shape == u.shape

