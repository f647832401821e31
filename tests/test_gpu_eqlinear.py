"""GPU parity of the group-axis circular convolution (fftconv_eqlinear_*) against
the CPU oracle (oracle.eqlinear: the plain definition, pinned in
test_oracle_eqlinear.py).  Inputs are seeded N(0, 1) activations and weights
N(0, 1 / (T C_in)); fp16 and bf16 storage; a token count that is not a
multiple of the 16-token tile; several output-channel spans."""
import sys

import numpy as np
import pytest
import torch

import long_fft_convolution_amd as fc
from oracle.eqlinear import eqlinear, eqlinear_tokens
from parity import check

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.float16: 5e-3, torch.bfloat16: 2e-2}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(N, T, Ci, Co, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((N, T, Ci), generator=g).to(dtype)
    W = (torch.randn((T, Co, Ci), generator=g) / np.sqrt(T * Ci)).to(dtype)
    return x, W


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("T,Ci,Co,N", [(8, 32, 32, 16), (8, 64, 96, 50), (4, 128, 64, 37),
                                       (8, 128, 256, 300), (16, 96, 32, 17), (16, 32, 64, 33)])
def test_eqlinear_parity(dtype, T, Ci, Co, N):
    _say(f"eqlinear {dtype} T={T} Ci={Ci} Co={Co} N={N}")
    x, W = _inputs(N, T, Ci, Co, dtype, seed=T * 1000 + Ci + Co + N)
    y = fc.eqlinear(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    ref = eqlinear(x.double().numpy(), W.double().numpy())
    check(y.float().cpu().double().numpy(), ref, TOL[dtype])


def test_eqlinear_equivariance_on_gpu():
    # shifting the group axis of the input shifts the output (exactly the same
    # arithmetic on permuted rows, so equal to rounding)
    x, W = _inputs(64, 8, 64, 64, torch.float16, seed=3)
    xs = torch.roll(x, 3, dims=1)
    y = fc.eqlinear(x.cuda(), W.cuda()).float().cpu()
    ys = fc.eqlinear(xs.cuda(), W.cuda()).float().cpu()
    check(ys.numpy(), torch.roll(y, 3, dims=1).numpy(), 5e-3)


def test_eqlinear_bench_shape_sampled():
    # the benchmark shape, checked on sampled tokens
    N, T, Ci, Co = 65536, 8, 128, 128
    _say(f"eqlinear N={N} sampled")
    x, W = _inputs(N, T, Ci, Co, torch.float16, seed=11)
    y = fc.eqlinear(x.cuda(), W.cuda()).float().cpu().double().numpy()
    toks = np.random.default_rng(0).choice(N, 300, replace=False)
    toks = np.concatenate([toks, [0, N - 1]])
    ref = eqlinear_tokens(x.double().numpy(), W.double().numpy(), toks)
    check(y[toks], ref, 5e-3)


def test_eqlinear_empty():
    x = torch.empty((0, 8, 32), dtype=torch.float16, device="cuda")
    W = torch.randn(8, 32, 32).to(torch.float16).cuda()
    assert fc.eqlinear(x, W).shape == (0, 8, 32)


def test_eqlinear_fp32_equivariance_and_bench_shape():
    # fp32 storage and arithmetic: the shift equivariance to fp32 rounding, and the
    # benchmark shape on sampled tokens
    x, W = _inputs(64, 8, 64, 96, torch.float32, seed=5)
    y = fc.eqlinear(x.cuda(), W.cuda()).cpu()
    ys = fc.eqlinear(torch.roll(x, 3, dims=1).cuda(), W.cuda()).cpu()
    check(ys.double().numpy(), torch.roll(y, 3, dims=1).double().numpy(), 1e-6)
    N, T, Ci, Co = 65536, 8, 128, 128
    _say(f"eqlinear fp32 N={N} sampled")
    x, W = _inputs(N, T, Ci, Co, torch.float32, seed=12)
    y = fc.eqlinear(x.cuda(), W.cuda()).cpu().double().numpy()
    toks = np.concatenate([np.random.default_rng(1).choice(N, 300, replace=False), [0, N - 1]])
    check(y[toks], eqlinear_tokens(x.double().numpy(), W.double().numpy(), toks), 1e-5)
