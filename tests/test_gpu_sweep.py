"""Seeded random-shape sweeps on the GPU against the oracle, for the paths whose
index arithmetic has the most cases: the N = 1024 matrix-core kernel (batch
pairs, channel ranges per XCD), its chunked short-filter windows, and the
backward pass at N = 1024 (fused dk, two-output du / dw call).  Plus the
short-filter benchmark workload at full size on sampled outputs.

Shapes are drawn from numpy.random.default_rng with fixed seeds, so every run
checks the same cases.
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
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(t):
    return None if t is None else t.cuda()


def _shape(rng):
    dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
    gates = ["both", "none", "w", "v"][int(rng.integers(0, 4))]
    return dtype, gates


def _drop(inp, gates):
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    return inp


def _f64(inp, name):
    t = getattr(inp, name)
    return None if t is None else inp.f64(name)


@pytest.mark.parametrize("case", range(6))
def test_sweep_short_filter(case):
    rng = np.random.default_rng(500 + case)
    dtype, gates = _shape(rng)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 12))
    N = 1024 * int(rng.integers(1, 13))
    L = int(rng.integers(1, 1025))
    _say(f"short sweep {case}: B={B} H={H} N={N} L={L} {dtype} gates={gates}")
    inp = _drop(synth.generate(B, H, N, L, dtype, gated=True, seed=600 + case), gates)
    y = fc.causal_conv_short(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v))
    torch.cuda.synchronize()
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), _f64(inp, "w"), _f64(inp, "v"))
    check(y.float().cpu().double().numpy(), ref, TOL[dtype])


@pytest.mark.parametrize("case", range(6))
def test_sweep_pair_forward(case):
    rng = np.random.default_rng(700 + case)
    dtype, gates = _shape(rng)
    B, H = int(rng.integers(1, 10)), int(rng.integers(1, 90))
    L = int(rng.integers(1, 1025))
    _say(f"pair sweep {case}: B={B} H={H} L={L} {dtype} gates={gates}")
    inp = _drop(synth.generate(B, H, 1024, L, dtype, gated=True, seed=800 + case), gates)
    y = fc.causal_conv(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v))
    torch.cuda.synchronize()
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), _f64(inp, "w"), _f64(inp, "v"))
    check(y.float().cpu().double().numpy(), ref, TOL[dtype])


@pytest.mark.parametrize("case", range(6))
def test_sweep_backward_n1024(case):
    rng = np.random.default_rng(900 + case)
    dtype, gates = _shape(rng)
    B, H = int(rng.integers(1, 8)), int(rng.integers(1, 40))
    L = int(rng.integers(1, 1025))
    masked = bool(rng.integers(0, 2))
    _say(f"bwd sweep {case}: B={B} H={H} L={L} {dtype} gates={gates} mask={masked}")
    inp = _drop(synth.generate(B, H, 1024, L, dtype, gated=True, seed=1000 + case), gates)
    g = torch.Generator().manual_seed(1100 + case)
    dy = torch.randn((B, H, 1024), generator=g, dtype=torch.float64).to(TDT[dtype])
    mask = synth.random_mask(H, seed=1200 + case) if masked else None
    m = None if mask is None else torch.from_numpy(mask).cuda()
    got = fc.causal_conv_bwd(_dev(inp.u), _dev(inp.k), _dev(dy), _dev(inp.w), _dev(inp.v), m)
    torch.cuda.synchronize()
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), _f64(inp, "w"), _f64(inp, "v"), mask)
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        check(a.float().cpu().double().numpy(), b, TOL[dtype], name)


def test_short_workload_sampled():
    # the short-filter benchmark workload whole on the GPU, checked at sampled outputs
    wl = synth.WORKLOADS["short_fp16_n1m_l512"]
    _say(f"short workload {wl.name} sampled")
    inp = synth.generate_workload(wl.name)
    y = fc.causal_conv_short(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v))
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    n = 400
    pts = np.stack([rng.integers(0, wl.B, n), rng.integers(0, wl.H, n), rng.integers(0, wl.N, n)], 1)
    edge = np.array([[0, 0, 0], [0, wl.H - 1, wl.N - 1], [0, 3, 1023], [0, 5, 1024], [0, 7, 2047], [0, 9, 2048]])
    pts = np.concatenate([pts, edge]).astype(np.int64)
    ref = oracle.direct_points(inp.f64("u"), inp.f64("k"), pts, _f64(inp, "w"), _f64(inp, "v"))
    yc = y.float().cpu().double().numpy()
    got = yc[pts[:, 0], pts[:, 1], pts[:, 2]]
    check(got, ref, TOL["f16"], "sampled outputs")
    # whole sequences: a seeded set of channels, every output against the exact sums
    hs = np.concatenate([[0, wl.H - 1], rng.choice(np.arange(1, wl.H - 1), 4, replace=False)])
    seq = lambda t: None if t is None else t[:, hs].to(torch.float64).numpy()
    ref_seq = oracle.fft_conv(seq(inp.u), inp.k[hs].to(torch.float64).numpy(), seq(inp.w), seq(inp.v))
    check(yc[:, hs], ref_seq, TOL["f16"], "whole sequences")
