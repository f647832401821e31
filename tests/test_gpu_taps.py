"""GPU parity of the forward call from time-domain taps (fftconv_fwd_taps).

The call transforms the (H, L) taps into a spectrum held in its workspace and runs
the forward kernels on it.  Each case checks that its output equals, bit for bit,
that of fftconv_prepare_filter followed by fftconv_fwd on the same inputs (the same
kernels in the same order), and compares it element by element with the oracle's
convolution of the rounded inputs (relative L2: 1e-5 fp32, 5e-3 fp16, 2e-2 bf16).
Sizes cover the on-chip kernels (N = 1024, 16384, the fused fp32 kernel) and the
multi-pass path, partial filters (L < N) and a frequency mask.
"""
import sys

import pytest
import torch

import oracle
import long_fft_convolution_amd as fc
from long_fft_convolution_amd import synth
from parity import check

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(t):
    return None if t is None else t.cuda()


def _taps(u, k, w, v, mask=None):
    B, H, N = u.shape
    ws = torch.empty(fc.fftconv_fwd_taps_workspace_bytes(B, H, N, u.dtype), dtype=torch.uint8, device=u.device)
    out = torch.empty_like(u)
    fc.fftconv_fwd_taps(u, k, w, v, out, ws, mask)
    return out


@pytest.mark.parametrize("dtype,B,H,N,L,gated", [
    ("f16", 4, 9, 1024, 300, True),          # pair kernel, N = 1024
    ("bf16", 3, 9, 16384, 5000, True),       # pair kernel, N = 16384, odd batch
    ("f32", 2, 3, 4096, 4096, True),         # fused fp32 kernel, full-length filter
    ("f16", 1, 3, 1 << 17, 2000, False),     # multi-pass path, short partial filter
    ("f32", 1, 2, 1 << 16, 1 << 14, True),   # multi-pass path, fp32
])
def test_taps_matches_prepared_and_oracle(dtype, B, H, N, L, gated):
    _say(f"taps {dtype} B={B} H={H} N={N} L={L} gated={gated}")
    inp = synth.generate(B, H, N, L, dtype, gated=gated, seed=N + L)
    u, k, w, v = _dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v)
    got = _taps(u, k, w, v)
    want_gpu = fc.causal_conv(u, k, w, v)
    torch.cuda.synchronize()
    assert torch.equal(got, want_gpu)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(got.float().cpu().double().numpy(), ref, TOL[dtype])


@pytest.mark.parametrize("dtype,N", [("f16", 1024), ("bf16", 16384), ("f16", 1 << 18)])
def test_taps_masked(dtype, N):
    H = 3
    _say(f"taps masked {dtype} N={N}")
    inp = synth.generate(2, H, N, N // 4, dtype, gated=False, seed=N + 5)
    mask = synth.random_mask(H, seed=N)
    m = torch.from_numpy(mask).cuda()
    u, k = _dev(inp.u), _dev(inp.k)
    got = _taps(u, k, None, None, m)
    want_gpu = fc.causal_conv(u, k, None, None, m)
    torch.cuda.synchronize()
    assert torch.equal(got, want_gpu)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), mask=mask)
    check(got.float().cpu().double().numpy(), ref, TOL[dtype])


def test_taps_repeated_calls_share_a_workspace():
    # a second call with other taps through the same workspace overwrites the spectrum
    B, H, N = 2, 4, 16384
    _say("taps repeated calls")
    a = synth.generate(B, H, N, 700, "f16", gated=True, seed=11)
    b = synth.generate(B, H, N, 9000, "f16", gated=True, seed=12)
    ws = torch.empty(fc.fftconv_fwd_taps_workspace_bytes(B, H, N, torch.float16), dtype=torch.uint8, device="cuda")
    outs = []
    for inp in (a, b):
        out = torch.empty(inp.u.shape, dtype=inp.u.dtype, device="cuda")
        fc.fftconv_fwd_taps(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v), out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    for inp, out in zip((a, b), outs):
        ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
        check(out.float().cpu().double().numpy(), ref, TOL["f16"])
