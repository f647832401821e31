"""GPU parity for inputs away from the N(0, 1) design point: non-zero means (the
zero-frequency bin of an unnormalised N-point transform grows to N times the
mean) and bf16 activations of large magnitude.  The half-precision kernels hold
their stage results in fp16; the power-of-two factors folded into their DFT
tables keep those results near the input's magnitude (for the bounds see the
header, fftconv.h).  Every case is compared with the oracle sequence by
sequence (tests/parity.check)."""
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


def _shift(t, loc, scale):
    """scale * t + loc, rounded back to t's storage type (the oracle reads the rounded values)."""
    return None if t is None else (t.double() * scale + loc).to(t.dtype)


def _run_and_check(inp, dtype, what, mask=None):
    dev = torch.device("cuda")
    d = lambda t: None if t is None else t.to(dev)
    m = None if mask is None else torch.from_numpy(mask).to(dev)
    y = fc.causal_conv(d(inp.u), d(inp.k), d(inp.w), d(inp.v), m)
    torch.cuda.synchronize()
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"), mask=mask)
    check(y.float().cpu().double().numpy(), ref, TOL[dtype], what)


@pytest.mark.parametrize("dtype,B,H,N,loc,gated", [
    ("bf16", 2, 3, 16384, 2.0, True),     # u, w ~ N(2, 1): mean(u w) = 4, DC = 65536 * 1 unscaled
    ("f16", 2, 3, 16384, 4.0, True),      # mean(u w) = 16
    ("f16", 4, 5, 1024, 8.0, True),       # mean(u w) = 64 at N = 1024
    ("bf16", 3, 4, 1024, 3.0, False),     # ungated, mean 3
    ("f16", 2, 3, 4096, 5.0, True),       # the fp32 fused kernel (fp16 storage)
])
def test_nonzero_mean_on_chip(dtype, B, H, N, loc, gated):
    _say(f"mean {loc} {dtype} B={B} H={H} N={N} gated={gated}")
    inp = synth.generate(B, H, N, N, dtype, gated=gated, seed=N + int(loc))
    inp.u = _shift(inp.u, loc, 1.0)
    inp.w = _shift(inp.w, loc, 1.0)
    _run_and_check(inp, dtype, f"mean {loc} N={N}")


@pytest.mark.parametrize("dtype,N,L,loc,masked", [
    ("f16", 1 << 20, 1 << 20, 0.5, False),   # u ~ N(0.5, 1) at N = 2^20
    ("f16", 1 << 22, 1 << 20, 0.5, True),    # the 4M partial workload's shape, masked
    ("bf16", 1 << 18, 1 << 18, 2.0, False),
    ("f16", 1 << 15, 1 << 15, 4.0, False),
])
def test_nonzero_mean_multipass(dtype, N, L, loc, masked):
    H = 2
    _say(f"multipass mean {loc} {dtype} N={N} masked={masked}")
    inp = synth.generate(1, H, N, L, dtype, gated=False, seed=N + 3,
                         mask_keep_blocks=27 if masked else None)
    inp.u = _shift(inp.u, loc, 1.0)
    _run_and_check(inp, dtype, f"multipass mean {loc} N={N}", inp.mask)


@pytest.mark.parametrize("N", [1024, 16384, 1 << 18])
@pytest.mark.parametrize("scale", [1e3, 1e-3])
def test_bf16_scaled_inputs(N, scale):
    # bf16 activations 1000x (and 1/1000x) the design scale; the gate w stays N(0, 1)
    _say(f"bf16 x{scale} N={N}")
    inp = synth.generate(2, 3, N, N, "bf16", gated=True, seed=N + 11)
    inp.u = _shift(inp.u, 0.0, scale)
    _run_and_check(inp, "bf16", f"bf16 u x {scale} N={N}")
