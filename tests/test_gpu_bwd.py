"""GPU parity of the backward pass against the oracle's backward routes.

Every case draws seeded inputs and an output gradient dy, rounds them to the
storage dtype, runs fftconv_bwd through the C ABI and compares du, dk, dw, dv
element by element with oracle.fft_bwd (oracle.direct_bwd at N = 1024) on the
rounded values.  Sizes cover each forward path the backward reuses: the
N = 1024 and N = 16384 matrix-core kernels (fp16 / bf16), the fused fp32
kernel and the multi-pass path.  Tolerances (relative L2 per gradient) as for
the forward pass: 1e-5 fp32, 5e-3 fp16, 2e-2 bf16.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import long_fft_convolution_amd as fc
from long_fft_convolution_amd import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _case(B, H, N, L, dtype, gates, seed):
    inp = synth.generate(B, H, N, L, dtype, gated=True, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    dy = torch.randn((B, H, N), generator=g, dtype=torch.float64).to(TDT[dtype])
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    return inp, dy


def _run(inp, dy, mask=None):
    dev = torch.device("cuda")
    m = None if mask is None else torch.from_numpy(mask).to(dev)
    d = lambda t: None if t is None else t.to(dev)
    res = fc.causal_conv_bwd(d(inp.u), d(inp.k), d(dy), d(inp.w), d(inp.v), m)
    torch.cuda.synchronize()
    return [None if t is None else t.float().cpu().double().numpy() for t in res]


def _check(got, want, tol):
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        err = oracle.rel_l2(a, b)
        assert err < tol, f"{name}: rel L2 {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gates", ["both", "none", "w", "v"])
def test_bwd_n1024(dtype, gates):
    B, H, N, L = 3, 2, 1024, 1024
    _say(f"bwd N={N} {dtype} gates={gates}")
    inp, dy = _case(B, H, N, L, dtype, gates, seed=71)
    got = _run(inp, dy)
    want = oracle.direct_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("dtype,N,L", [("f32", 2048, 2048), ("f16", 4096, 1000), ("bf16", 16384, 16384),
                                       ("f16", 16384, 3000), ("f32", 1 << 15, 1 << 15),
                                       ("f16", 1 << 15, 5000), ("bf16", 1 << 16, 1 << 16)])
def test_bwd_sizes(dtype, N, L):
    B, H = 2, 2
    _say(f"bwd N={N} L={L} {dtype}")
    inp, dy = _case(B, H, N, L, dtype, "both", seed=N + L)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("dtype,N", [("f32", 1024), ("f16", 1024), ("bf16", 16384), ("f32", 1 << 15)])
@pytest.mark.parametrize("kind", ["band", "random"])
def test_bwd_mask(dtype, N, kind):
    B, H = 2, 3
    _say(f"bwd mask {kind} N={N} {dtype}")
    inp, dy = _case(B, H, N, N, dtype, "both", seed=N + 7)
    mask = synth.band_mask(H, 27) if kind == "band" else synth.random_mask(H, seed=N)
    got = _run(inp, dy, mask)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"), mask)
    _check(got, want, TOL[dtype])


def test_bwd_odd_batch_and_one_sequence():
    # B = 1: the matrix-core kernels pair a sequence with zeros; B = 5: odd tail
    for B in (1, 5):
        _say(f"bwd B={B}")
        inp, dy = _case(B, 2, 1024, 1024, "f16", "both", seed=B)
        got = _run(inp, dy)
        want = oracle.direct_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
        _check(got, want, TOL["f16"])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_n1024_many_channels(dtype):
    # N = 1024: dk comes from one kernel per channel; more channels than CUs (a workgroup
    # walks several), an odd batch, a filter shorter than the sequence
    B, H, N, L = 5, 300, 1024, 700
    _say(f"bwd N={N} B={B} H={H} L={L} {dtype}")
    inp, dy = _case(B, H, N, L, dtype, "both", seed=301)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("gates", ["w", "both"])
def test_bwd_n16384_channels(gates):
    # N = 16384: du and dw come from one kernel call; an odd batch (the last pair has one
    # sequence), enough channels for the per-XCD channel split, with and without the
    # input gate v
    B, H, N = 3, 9, 16384
    _say(f"bwd N={N} B={B} H={H} gates={gates}")
    inp, dy = _case(B, H, N, N, "f16", gates, seed=163)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL["f16"])


def test_bwd_workload_full_size():
    # the backward benchmark's configuration (gated_fp16_n1k: B = 64, H = 768, N = 1024,
    # the same dy recipe), every gradient compared whole against the oracle
    wl = synth.WORKLOADS["gated_fp16_n1k"]
    _say(f"bwd {wl.name} full size")
    inp = synth.generate_workload(wl.name)
    g = torch.Generator().manual_seed(4242)
    dy = torch.randn(inp.u.shape, generator=g, dtype=torch.float32).to(inp.u.dtype)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL["f16"])
