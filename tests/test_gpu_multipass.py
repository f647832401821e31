"""GPU parity of the multi-pass path (N > 16384) against the CPU oracle.

Sizes span every outer length N1 = N / 8192 from 4 to 512 at small B*H so the
oracle's float64 FFT route finishes in seconds; chunking over sequences is
exercised by B*H larger than one chunk.  Tolerances as in the fused tests.
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

TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(t):
    return None if t is None else t.cuda()


def run_gpu(inp, mask=None):
    m = None if mask is None else torch.from_numpy(mask).cuda()
    y = fc.causal_conv(_dev(inp.u), _dev(inp.k), _dev(inp.w), _dev(inp.v), m)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


@pytest.mark.parametrize("logn", [15, 16, 17, 18, 19, 20])
def test_multipass_sizes_fp32(logn):
    N = 1 << logn
    _say(f"multipass fp32 N={N}")
    inp = synth.generate(1, 2, N, N, "f32", gated=True, seed=logn)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multipass_half_dtypes(dtype):
    N = 1 << 17
    _say(f"multipass {dtype} N={N}")
    inp = synth.generate(2, 3, N, N, dtype, gated=True, seed=3)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("logn", [15, 16, 17, 18, 19, 20])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multipass_sizes_half(logn, dtype):
    # half-precision storage runs the row pass on the matrix cores: every outer
    # length N1 = 4 .. 128, gated
    N = 1 << logn
    _say(f"multipass {dtype} N={N}")
    inp = synth.generate(1, 3, N, N, dtype, gated=True, seed=100 + logn)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("logn,H", [(21, 2), (22, 2), (21, 17)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multipass_matrix_core_columns(logn, H, dtype):
    # N1 = 256 and 512: both column passes on the matrix cores, gated, every sequence
    # compared whole; H = 17 at N = 2^21 leaves a ragged last chunk (16 sequences per chunk)
    N = 1 << logn
    _say(f"multipass columns {dtype} N={N} H={H}")
    inp = synth.generate(1, H, N, N if H == 2 else 1 << 12, dtype, gated=True, seed=200 + logn + H)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("kind", ["band", "random"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multipass_mask_half(kind, dtype):
    N = 1 << 18
    _say(f"multipass mask {kind} {dtype}")
    inp = synth.generate(1, 3, N, 1 << 16, dtype, gated=False, seed=19)
    mask = synth.band_mask(3, 27) if kind == "band" else synth.random_mask(3, seed=15)
    y = run_gpu(inp, mask)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), mask=mask)
    check(y, ref, TOL[dtype])


def test_multipass_chunks_half_ragged():
    # 2^16 points per sequence in fp16: 512 sequences per 128 MiB chunk; 515 -> a ragged chunk
    N = 1 << 16
    assert fc.fftconv_workspace_bytes(1, 515, N, torch.float16) == 512 * (N * 4 + 2 * 8192 * 8)
    _say("multipass chunking f16 B=1 H=515")
    inp = synth.generate(1, 515, N, 2048, "f16", gated=False, seed=24)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"))
    check(y, ref, TOL["f16"])


def test_multipass_chunks_and_ragged_tail():
    # 2^17 points per sequence in fp32: 128 sequences per 128 MiB chunk;
    # 131 sequences -> a ragged chunk
    N = 1 << 17
    assert fc.fftconv_workspace_bytes(1, 131, N, torch.float32) == 128 * (N * 8 + 2 * 8192 * 8)
    _say("multipass chunking B=1 H=131")
    inp = synth.generate(1, 131, N, 4096, "f32", gated=False, seed=4)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"))
    check(y, ref, TOL["f32"])


@pytest.mark.parametrize("L", [1, 777, 1 << 15])
def test_multipass_partial_filter(L):
    N = 1 << 16
    _say(f"multipass partial L={L}")
    inp = synth.generate(1, 2, N, L, "f32", gated=False, seed=L)
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"))
    check(y, ref, TOL["f32"])


@pytest.mark.parametrize("kind", ["band", "random"])
def test_multipass_mask(kind):
    N = 1 << 18
    _say(f"multipass mask {kind}")
    inp = synth.generate(1, 3, N, 1 << 16, "f32", gated=False, seed=9)
    mask = synth.band_mask(3, 27) if kind == "band" else synth.random_mask(3, seed=5)
    y = run_gpu(inp, mask)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), mask=mask)
    check(y, ref, TOL["f32"])


def test_multipass_prepared_spectrum():
    N = 1 << 20
    _say("multipass export K_f")
    inp = synth.generate(1, 2, N, 300000, "f16", seed=10)
    k = inp.k.cuda()
    K_f = fc.alloc_filter(2, N, k.dtype)
    ws = fc.alloc_workspace(1, 2, N, k.dtype)
    fc.fftconv_prepare_filter(k, N, K_f, ws)
    got = fc.fftconv_export_filter_rfft(K_f, 2, N, k.dtype)
    k64 = inp.f64("k")
    for h in range(2):
        x = np.zeros(2 * N, complex)
        x[:k64.shape[1]] = k64[h]
        want = oracle.fft(x)[:N + 1]
        assert np.linalg.norm(got[h] - want) / np.linalg.norm(want) < 2e-3


def test_multipass_largest_size_masked_partial():
    N = 1 << 22
    _say("multipass N=2^22 partial + band mask, H=2")
    inp = synth.generate(1, 2, N, 1 << 20, "f16", gated=False, seed=11, mask_keep_blocks=27)
    y = run_gpu(inp, inp.mask)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), mask=inp.mask)
    check(y, ref, TOL["f16"])


@pytest.mark.parametrize("keep", [(0, 27), (40, 88), (0, 128), (100, 128)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multipass_band_masks_half(keep, dtype):
    # contiguous kept bands: low (the 79 % mask: the row pass skips its middle-frequency
    # tile), middle (it skips the other tile), all (nothing skipped), high
    N, H = 1 << 19, 3
    lo, hi = keep
    _say(f"multipass band mask {lo}..{hi} {dtype}")
    inp = synth.generate(1, H, N, 1 << 17, dtype, gated=False, seed=lo + hi)
    mask = np.zeros((H, 128), dtype=np.uint8)
    mask[:, lo:hi] = 1
    y = run_gpu(inp, mask)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), mask=mask)
    check(y, ref, TOL[dtype])
