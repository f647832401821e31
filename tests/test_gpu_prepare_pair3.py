"""GPU parity of the filter prepare at N = 2048 .. 16384 in fp16 / bf16 storage, which
runs the forward transform of the N = 16384 matrix-core kernels (its R-row variant below
16384) on each channel's zero-padded taps and stores K s_h (rows f_c <= R/2 of the
KF_PAIR3 layout), the taps entering scaled by s_h 2^14.

Each prepared spectrum is decoded to natural-order rfft bins and compared per channel
with the oracle's 2N-point FFT of the rounded taps (relative L2 per channel).  The cases:
every size, odd and edge filter lengths (1, 7, N - 1, N), channel counts that leave the
last channel group partial, filters scaled by 1e-6 and 1e3 (the power-of-two pre-scale
keeps small taps out of fp16's subnormal range), an all-zero channel (exactly zero bins,
its neighbours exact), and the forward call through such a filter against direct sums.
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

# relative L2 of one channel's spectrum: three fp16-rounded stages and the fp16 store
SPEC_TOL = 2e-3
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
# channels per workgroup group of the R-row variant (P = 32 / R, R = 2N / 1024)
P_OF = {2048: 8, 4096: 4, 8192: 2, 16384: 1}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _prepared(k, N):
    H = k.shape[0]
    K_f = fc.alloc_filter(H, N, k.dtype)
    fc.fftconv_prepare_filter(k, N, K_f)
    return fc.fftconv_export_filter_rfft(K_f, H, N, k.dtype)


def _want(k64, N):
    H, L = k64.shape
    out = np.empty((H, N + 1), complex)
    for h in range(H):
        x = np.zeros(2 * N, complex)
        x[:L] = k64[h]
        out[h] = oracle.fft(x)[:N + 1]
    return out


def _check_channels(got, want, tol=SPEC_TOL):
    for h in range(want.shape[0]):
        nw = np.linalg.norm(want[h])
        if nw == 0.0:
            assert np.all(got[h] == 0), f"channel {h}: zero taps, non-zero bins"
            continue
        err = np.linalg.norm(got[h] - want[h]) / nw
        assert err < tol, f"channel {h}: relative L2 {err:.2e}"


def _taps(H, L, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    decay = torch.exp(-torch.arange(L, dtype=torch.float64) * (4.0 / L))
    k = torch.randn((H, L), generator=g, dtype=torch.float64) * decay * scale
    return k.to(TDT[dtype])


@pytest.mark.parametrize("N", [2048, 4096, 8192, 16384])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Lsel", ["one", "odd", "short", "n_minus_1", "full"])
def test_prepare_spectrum(N, dtype, Lsel):
    L = {"one": 1, "odd": 7, "short": 1000, "n_minus_1": N - 1, "full": N}[Lsel]
    H = 2 * P_OF[N] + 1   # a partial last channel group
    _say(f"prepare N={N} {dtype} L={L} H={H}")
    k = _taps(H, L, dtype, seed=N + L)
    got = _prepared(k.cuda(), N)
    _check_channels(got, _want(k.double().numpy(), N))


@pytest.mark.parametrize("N", [2048, 16384])
@pytest.mark.parametrize("scale", [1e-6, 1e3])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prepare_filter_scale(N, scale, dtype):
    # |k| ~ 1e-6 lies below fp16's normal range before the power-of-two pre-scale
    H, L = P_OF[N] + 1, N
    _say(f"prepare scale {scale} N={N} {dtype}")
    k = _taps(H, L, dtype, seed=17, scale=scale)
    got = _prepared(k.cuda(), N)
    _check_channels(got, _want(k.double().numpy(), N))


@pytest.mark.parametrize("N", [2048, 8192, 16384])
def test_prepare_zero_channel(N):
    H = P_OF[N] + 2
    _say(f"prepare zero channel N={N}")
    k = _taps(H, 500, "f16", seed=23)
    k[1] = 0
    got = _prepared(k.cuda(), N)
    _check_channels(got, _want(k.double().numpy(), N))


@pytest.mark.parametrize("N,L,H,B", [(2048, 333, 9, 3), (4096, 777, 9, 2), (8192, 8191, 5, 1), (16384, 5000, 3, 2)])
def test_forward_through_prepared_filter(N, L, H, B):
    _say(f"forward through the prepared filter N={N} L={L} H={H} B={B}")
    inp = synth.generate(B, H, N, L, "bf16", gated=True, seed=N + H)
    d = lambda t: None if t is None else t.cuda()
    y = fc.causal_conv(d(inp.u), d(inp.k), d(inp.w), d(inp.v))
    torch.cuda.synchronize()
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y.float().cpu().double().numpy(), ref, 2e-2)
