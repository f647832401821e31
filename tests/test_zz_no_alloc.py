"""fftconv_fwd_noalloc (the forward call for callers that cannot allocate)
against fftconv_fwd, through the C ABI: two calls in a row on one device, the
second with a smaller input, each equal to fftconv_fwd's output bit for bit
(the same kernels per sequence; only the chunking of the three-pass path
through the scratch differs) and within the storage type's tolerance of the
oracle."""
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


def _both(inp, L, masked):
    dev = torch.device("cuda")
    u, k = inp.u.to(dev), inp.k.to(dev)
    w = None if inp.w is None else inp.w.to(dev)
    v = None if inp.v is None else inp.v.to(dev)
    B, H, N = u.shape
    mask = torch.from_numpy(synth.random_mask(H, seed=N)).to(dev) if masked else None
    K_f = fc.alloc_filter(H, N, u.dtype, dev)
    fc.fftconv_prepare_filter(k, N, K_f, fc.alloc_workspace(1, H, N, u.dtype, dev))
    want = torch.empty_like(u)
    fc.fftconv_fwd(u, K_f, w, v, want, L, mask, fc.alloc_workspace(B, H, N, u.dtype, dev))
    got = torch.full_like(u, float("nan"))
    fc.fftconv_fwd_noalloc(u, K_f, w, v, got, L, mask)
    torch.cuda.synchronize()
    return got, want, mask


def test_noalloc_two_calls_second_smaller():
    fc.fftconv_init()
    assert fc.fftconv_fwd_noalloc_scratch_bytes() == 72 << 20
    # call 1: N = 2^22 fp16, 6 sequences -> two chunks of the 72 MiB scratch (4 + 2)
    # call 2: N = 2^18 bf16, gated, masked, 3 sequences -> one chunk
    # call 3: N = 1024 fp16 (no scratch: the on-chip kernel)
    cases = [(1, 6, 1 << 22, 1 << 20, "f16", False, False),
             (1, 3, 1 << 18, 5000, "bf16", True, True),
             (2, 3, 1024, 1024, "f16", True, False)]
    for B, H, N, L, dtype, gated, masked in cases:
        _say(f"noalloc B={B} H={H} N={N} L={L} {dtype} gated={gated} masked={masked}")
        inp = synth.generate(B, H, N, L, dtype, gated=gated, seed=N + H)
        got, want, mask = _both(inp, L, masked)
        assert torch.equal(got, want), "fftconv_fwd_noalloc differs from fftconv_fwd"
        m = None if mask is None else mask.cpu().numpy()
        ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"), mask=m)
        check(got.float().cpu().double().numpy(), ref, TOL[dtype], f"noalloc N={N}")


def test_noalloc_needs_init_on_the_device_and_checks_arguments():
    fc.fftconv_init()
    u = torch.zeros((1, 2, 1000), dtype=torch.float16, device="cuda")
    K_f = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fc.FFTConvError) as e:
        fc.fftconv_fwd_noalloc(u, K_f, None, None, torch.empty_like(u), 1000)
    assert e.value.status == 2   # N = 1000: unsupported size
