"""GPU parity of the last batch row of an odd B at N = 1024 (fp16 / bf16), which the
N = 1024 kernel packs as channel pairs (h, h + 1) instead of pairing each of its
sequences with zeros: z = x_h + i x_h', the product Y(f) = Z(f) (K + K') / 2 +
conj Z(-f) (K - K') / 2, the real part scaled as channel h and the imaginary part
as channel h'.  Every case is checked per sequence against the oracle: B = 1 and
B = 3, even and odd H (the last channel without a partner), every gate
combination, per-channel frequency masks, two channels of one pair whose filter
scales and input magnitudes differ by orders of magnitude, and the backward pass
(the two-output kernel for du and dw) with B = 1.
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


def _d(t):
    return None if t is None else t.cuda()


def _fwd(inp, mask=None):
    m = None if mask is None else torch.from_numpy(mask).cuda()
    y = fc.causal_conv(_d(inp.u), _d(inp.k), _d(inp.w), _d(inp.v), m)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _gates(inp, gates):
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    return inp


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B,H", [(1, 2), (1, 3), (1, 8), (3, 5), (1, 1)])
@pytest.mark.parametrize("gates", ["none", "w", "v", "both"])
def test_lone_row_channel_pairs(dtype, B, H, gates):
    _say(f"lone row {dtype} B={B} H={H} gates={gates}")
    inp = _gates(synth.generate(B, H, 1024, 900, dtype, gated=True, seed=10 * B + H), gates)
    y = _fwd(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("kind", ["band", "random"])
@pytest.mark.parametrize("H", [4, 5])
def test_lone_row_masks(kind, H):
    # each channel of a pair has its own mask row
    _say(f"lone row mask {kind} H={H}")
    inp = synth.generate(1, H, 1024, 1024, "f16", gated=True, seed=40 + H)
    mask = synth.band_mask(H, 27) if kind == "band" else synth.random_mask(H, seed=H)
    y = _fwd(inp, mask)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"), mask=mask)
    check(y, ref, TOL["f16"])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_lone_row_unequal_channels(dtype):
    # the two channels of a pair with filters 10^3 apart and inputs 10^2 apart: each
    # sequence is checked against its own norm, so a leak of one channel into the other
    # (or the wrong channel scale) fails
    _say(f"lone row unequal channels {dtype}")
    inp = synth.generate(1, 4, 1024, 1024, dtype, gated=True, seed=77)
    k = inp.k.double()
    k[0] *= 30.0
    k[1] *= 0.03
    k[3] *= 1e-2
    inp.k = k.to(inp.k.dtype)
    u = inp.u.double()
    u[:, 1] *= 1e-2
    u[:, 2] *= 10.0
    inp.u = u.to(inp.u.dtype)
    y = _fwd(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("H,gates", [(3, "both"), (3, "w"), (4, "none"), (4, "v")])
def test_lone_row_backward(H, gates):
    # B = 1: du and dw from the two-output channel-pair kernel, dv from the forward one
    _say(f"lone row backward H={H} gates={gates}")
    inp = _gates(synth.generate(1, H, 1024, 1024, "f16", gated=True, seed=90 + H), gates)
    g = torch.Generator().manual_seed(91 + H)
    dy = torch.randn((1, H, 1024), generator=g, dtype=torch.float64).to(torch.float16)
    res = fc.causal_conv_bwd(_d(inp.u), _d(inp.k), _d(dy), _d(inp.w), _d(inp.v))
    torch.cuda.synchronize()
    got = [None if t is None else t.float().cpu().double().numpy() for t in res]
    want = oracle.direct_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(),
                             None if inp.w is None else inp.f64("w"), None if inp.v is None else inp.f64("v"))
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        check(a, b, TOL["f16"], name)


def test_lone_row_matches_noalloc():
    # the same rows through fftconv_fwd_noalloc (the same launches, bit-equal), B = 3
    _say("lone row vs noalloc")
    fc.fftconv_init()
    inp = synth.generate(3, 6, 1024, 1024, "f16", gated=True, seed=123)
    u, k, w, v = (_d(t) for t in (inp.u, inp.k, inp.w, inp.v))
    K = fc.alloc_filter(6, 1024, u.dtype, u.device)
    fc.fftconv_prepare_filter(k, 1024, K, fc.alloc_workspace(1, 6, 1024, u.dtype, u.device))
    y1 = torch.empty_like(u)
    y2 = torch.empty_like(u)
    fc.fftconv_fwd(u, K, w, v, y1, 1024)
    fc.fftconv_fwd_noalloc(u, K, w, v, y2, 1024)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y1.float().cpu().double().numpy(), ref, TOL["f16"])
