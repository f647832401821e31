"""GPU checks that a sequence whose input x = u * w is all zero gets an output of
exactly zero on the matrix-core kernels (N = 1024 .. 16384, fp16 / bf16).

Those kernels transform two sequences as one complex sequence (two batch rows of
a channel, or at N = 2048 .. 8192 also several channels per workgroup); every
stage rounds at the magnitude of the larger one, so without a check a zero
sequence would come out as the rounding of its partner's values.  The cases: a
whole zero batch row, a single zero sequence inside a channel group, a zero gate
w, the last row of an odd batch (channel pairs at N = 1024), and the backward
pass's du and dw for a zero output gradient row.  The non-zero sequences are
checked against the oracle per sequence.
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


def _d(t):
    return None if t is None else t.cuda()


def _run(inp):
    y = fc.causal_conv(_d(inp.u), _d(inp.k), _d(inp.w), _d(inp.v))
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _ref(inp):
    N = inp.u.shape[-1]
    if N <= 2048:
        return oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    return oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))


def _check_zero_and_rest(y, ref, zero, tol):
    # zero: boolean (B, H) of the sequences whose input is zero
    assert np.all(y[zero] == 0.0), "a zero input sequence has a non-zero output"
    check(y[~zero], ref[~zero], tol)


@pytest.mark.parametrize("N", [1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_batch_row(N, dtype):
    _say(f"zero batch row N={N} {dtype}")
    inp = synth.generate(2, 3, N, N, dtype, gated=True, seed=N + 1)
    u = inp.u.clone()
    u[1] = 0
    inp.u = u
    zero = np.zeros((2, 3), dtype=bool)
    zero[1] = True
    _check_zero_and_rest(_run(inp), _ref(inp), zero, TOL[dtype])


@pytest.mark.parametrize("N,B,H", [(2048, 2, 9), (4096, 3, 5), (8192, 2, 3), (1024, 3, 4), (16384, 2, 2)])
def test_zero_single_sequence(N, B, H):
    # one sequence of the batch row pair (or of a channel group) is zero; its partner and
    # the group's other channels are not
    _say(f"zero single sequence N={N} B={B} H={H}")
    inp = synth.generate(B, H, N, N, "f16", gated=True, seed=N + 2)
    u = inp.u.clone()
    u[1, H // 2] = 0
    u[B - 1, H - 1] = 0
    inp.u = u
    zero = np.zeros((B, H), dtype=bool)
    zero[1, H // 2] = True
    zero[B - 1, H - 1] = True
    _check_zero_and_rest(_run(inp), _ref(inp), zero, TOL["f16"])


@pytest.mark.parametrize("N", [1024, 4096, 16384])
def test_zero_gate(N):
    # u non-zero but the input gate w zero: x = u * w = 0
    _say(f"zero gate N={N}")
    inp = synth.generate(2, 2, N, N, "bf16", gated=True, seed=N + 3)
    w = inp.w.clone()
    w[0, 1] = 0
    inp.w = w
    zero = np.zeros((2, 2), dtype=bool)
    zero[0, 1] = True
    _check_zero_and_rest(_run(inp), _ref(inp), zero, TOL["bf16"])


@pytest.mark.parametrize("N", [1024, 16384])
def test_zero_gradient_row(N):
    # dy zero for one sequence: its du and dw are exactly zero (v dy = 0)
    B, H = 2, 3
    _say(f"zero gradient row N={N}")
    inp = synth.generate(B, H, N, N, "f16", gated=True, seed=N + 4)
    g = torch.Generator().manual_seed(N + 5)
    dy = torch.randn((B, H, N), generator=g, dtype=torch.float64).to(torch.float16)
    dy[1, 2] = 0
    res = fc.causal_conv_bwd(_d(inp.u), _d(inp.k), _d(dy), _d(inp.w), _d(inp.v))
    torch.cuda.synchronize()
    du, dk, dw, dv = [t.float().cpu().double().numpy() for t in res]
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    zero = np.zeros((B, H), dtype=bool)
    zero[1, 2] = True
    for name, a, b in (("du", du, want[0]), ("dw", dw, want[2])):
        assert np.all(a[zero] == 0.0), name
        check(a[~zero], b[~zero], TOL["f16"], name)
    check(dk, want[1], TOL["f16"], "dk")
    check(dv, want[3], TOL["f16"], "dv")
