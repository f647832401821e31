"""GPU parity of the short-filter backward pass (fftconv_bwd_short) against the
oracle's backward routes.

fftconv_bwd_short forms dv with the windowed forward kernel (dy as the output
gate), corr(v dy, k) for du and dw with the correlation mode of that kernel
(the window of blocks j and j + 1, the conjugated spectrum, the first half of
the outputs), and dk with the windowed mode of the on-chip dk kernel.  Every
case rounds seeded inputs and dy to the storage dtype and compares du, dk, dw,
dv with oracle.direct_bwd (direct sums, any N) or oracle.fft_bwd (2N-point FFT,
long power-of-two N) on the rounded values.  The cases cover the first and last
windows (zeros before and past the sequence), the longest filter and a
one-tap filter, odd window counts (a last window pair with one window),
lengths that are multiples of 1024 but not powers of two, every gate
combination, single gradients (the one-output correlation kernels, equal to
the two-output one bit for bit), batch rows, more channels than one channel
per workgroup, an empty batch, and the full-size short-filter configuration
on a subset of its channels.  Tolerances as for the forward pass (relative L2
per gradient): 5e-3 fp16, 2e-2 bf16.
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


def _case(B, H, N, L, dtype, gates, seed):
    inp = synth.generate(B, H, N, L, dtype, gated=True, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    dy = torch.randn((B, H, N), generator=g, dtype=torch.float64).to(TDT[dtype])
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    return inp, dy


def _np(t):
    return None if t is None else t.float().cpu().double().numpy()


def _run(inp, dy):
    d = lambda t: None if t is None else t.cuda()
    res = fc.causal_conv_short_bwd(d(inp.u), d(inp.k), d(dy), d(inp.w), d(inp.v))
    torch.cuda.synchronize()
    return [_np(t) for t in res]


def _ref(inp, dy):
    w = None if inp.w is None else inp.f64("w")
    v = None if inp.v is None else inp.f64("v")
    N = inp.u.shape[-1]
    dyd = dy.double().numpy()
    if N & (N - 1) == 0 and N > 16384:
        return oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dyd, w, v)
    return oracle.direct_bwd(inp.f64("u"), inp.f64("k"), dyd, w, v)


def _check(got, want, tol):
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        check(a, b, tol, name)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,L", [(1024, 512), (1024, 1024), (2048, 1), (3072, 100), (3072, 1024),
                                 (5 * 1024, 257), (8192, 1023), (7 * 1024, 1000)])
def test_short_bwd_sizes(dtype, N, L):
    _say(f"short bwd {dtype} N={N} L={L} B=3 H=2")
    inp, dy = _case(3, 2, N, L, dtype, "both", seed=N + 7 * L)
    _check(_run(inp, dy), _ref(inp, dy), TOL[dtype])


@pytest.mark.parametrize("gates", ["none", "w", "v", "both"])
def test_short_bwd_gates(gates):
    N, L = 4096, 300
    _say(f"short bwd gates={gates} N={N}")
    inp, dy = _case(2, 3, N, L, "f16", gates, seed=11)
    _check(_run(inp, dy), _ref(inp, dy), TOL["f16"])


def test_short_bwd_single_gradients():
    # each gradient alone (the one-output correlation kernels for du and dw) equals the
    # same gradient of the full call bit for bit
    N, L, B, H = 5 * 1024, 700, 2, 3
    _say(f"short bwd single gradients N={N}")
    inp, dy = _case(B, H, N, L, "bf16", "both", seed=19)
    dev = torch.device("cuda")
    u, w, v, k, dyc = (t.to(dev) for t in (inp.u, inp.w, inp.v, inp.k, dy))
    K_s = torch.empty(fc.fftconv_short_filter_bytes(H, u.dtype), dtype=torch.uint8, device=dev)
    fc.fftconv_prepare_short_filter(k, K_s)
    full = [torch.empty_like(u), torch.empty((H, L), dtype=u.dtype, device=dev), torch.empty_like(u),
            torch.empty_like(u)]
    fc.fftconv_bwd_short(dyc, u, K_s, w, v, *full, L)
    for i, name in enumerate(("du", "dk", "dw", "dv")):
        outs = [None] * 4
        outs[i] = torch.full_like(full[i], 7.0)
        fc.fftconv_bwd_short(dyc, u, K_s, w, v, *outs, L)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], full[i]), name
    _check([_np(t) for t in full], _ref(inp, dy), TOL["bf16"])


def test_short_bwd_channels_and_rows():
    # H = 300 channels on 256 workgroups (some walk two channels), B = 3 rows in one
    # channel's pair list, 3 windows per sequence (a last pair with one window)
    N, L, B, H = 3072, 300, 3, 300
    _say(f"short bwd B={B} H={H} N={N}")
    inp, dy = _case(B, H, N, L, "f16", "both", seed=23)
    _check(_run(inp, dy), _ref(inp, dy), TOL["f16"])


def test_short_bwd_long_sequence():
    N, L = 1 << 20, 1024
    _say(f"short bwd N={N} L={L} B=1 H=2")
    inp, dy = _case(1, 2, N, L, "f16", "both", seed=29)
    _check(_run(inp, dy), _ref(inp, dy), TOL["f16"])


def test_short_bwd_matches_full_path():
    # the same gradients through the full-length spectrum (fftconv_bwd)
    N, L = 1 << 15, 512
    _say(f"short bwd vs full N={N}")
    inp, dy = _case(2, 2, N, L, "f16", "both", seed=31)
    got = _run(inp, dy)
    d = lambda t: None if t is None else t.cuda()
    full = [_np(t) for t in fc.causal_conv_bwd(d(inp.u), d(inp.k), d(dy), d(inp.w), d(inp.v))]
    torch.cuda.synchronize()
    want = _ref(inp, dy)
    _check(got, want, TOL["f16"])
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, full):
        check(a, b, 2 * TOL["f16"], f"{name} short vs full")


def test_short_bwd_empty_batch():
    H, L = 3, 64
    u = torch.empty((0, H, 2048), dtype=torch.float16, device="cuda")
    k = torch.randn(H, L).to(torch.float16).cuda()
    K_s = torch.empty(fc.fftconv_short_filter_bytes(H, u.dtype), dtype=torch.uint8, device="cuda")
    fc.fftconv_prepare_short_filter(k, K_s)
    dk = torch.full((H, L), 5.0, dtype=u.dtype, device="cuda")
    fc.fftconv_bwd_short(u, u, K_s, None, None, None, dk, None, None, L)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0


def test_short_bwd_workload_full_size():
    # the short-filter benchmark configuration (B = 1, H = 256, N = 2^20, 512 taps) run whole;
    # every gradient of 6 channels spread over the range compared with the oracle run on
    # those channels alone
    wl = synth.WORKLOADS["short_fp16_n1m_l512"]
    _say(f"short bwd {wl.name} full size")
    inp = synth.generate_workload(wl.name)
    g = torch.Generator().manual_seed(5151)
    dy = torch.randn(inp.u.shape, generator=g, dtype=torch.float32).to(inp.u.dtype)
    got = _run(inp, dy)
    hs = np.array([0, 1, 100, 128, 254, 255])
    sub = lambda t: t[:, hs]
    want = oracle.fft_bwd(sub(inp.f64("u")), inp.f64("k")[hs], sub(dy.double().numpy()))
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        check(a[hs] if name == "dk" else a[:, hs], b, TOL["f16"], f"{name} channels {list(hs)}")
