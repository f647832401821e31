"""GPU parity of the fused path (N <= 16384) against the CPU oracle.

Every case draws seeded inputs (long_fft_convolution_amd.synth), rounds them
to the storage dtype, runs the HIP library through its C ABI and compares,
element by element, with the oracle on exactly the rounded values.
Tolerances (relative L2 over the compared elements): 1e-5 fp32, 5e-3 fp16,
2e-2 bf16.
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


def _to_dev(t):
    return None if t is None else t.cuda()


def run_gpu(inp, mask=None):
    u, k, w, v = _to_dev(inp.u), _to_dev(inp.k), _to_dev(inp.w), _to_dev(inp.v)
    m = None if mask is None else torch.from_numpy(mask).cuda()
    y = fc.causal_conv(u, k, w, v, m)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def oracle_full(inp, mask=None):
    return oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"), mask=mask)


@pytest.mark.parametrize("logn", [10, 11, 12, 13, 14])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_fused_sizes_dtypes_ragged(logn, dtype):
    N = 1 << logn
    B, H = 3, 5                         # 15 sequences: a ragged last workgroup at every size
    _say(f"fused N={N} dtype={dtype} B={B} H={H} gated")
    inp = synth.generate(B, H, N, N, dtype, gated=True, seed=logn * 10 + len(dtype))
    y = run_gpu(inp)
    ref = oracle_full(inp)
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("L", [1, 17, 1000, 1024])
def test_fused_partial_filters_fp32(L):
    _say(f"fused partial L={L}")
    inp = synth.generate(2, 3, 1024, L, "f32", gated=False, decay="fixed0.01", seed=L)
    y = run_gpu(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"))
    check(y, ref, 1e-5)


def test_small_fp32_workload_full():
    _say("ungated_fp32_n1k full")
    inp = synth.generate_workload("ungated_fp32_n1k")
    y = run_gpu(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"))
    check(y, ref, 1e-5)
    assert np.max(np.abs(y - ref)) < 1e-4 * np.max(np.abs(ref))


@pytest.mark.parametrize("side", ["w", "v"])
def test_one_sided_gate(side):
    _say(f"one-sided gate {side}")
    inp = synth.generate(2, 3, 2048, 2048, "f32", gated=True, seed=5)
    if side == "w":
        inp.v = None
    else:
        inp.w = None
    y = run_gpu(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, 1e-5)


@pytest.mark.parametrize("logn", [10, 14])
@pytest.mark.parametrize("kind", ["band", "random"])
def test_fused_frequency_mask(logn, kind):
    N = 1 << logn
    _say(f"mask {kind} N={N}")
    inp = synth.generate(2, 3, N, N, "f32", gated=True, seed=7)
    mask = synth.band_mask(3, 27) if kind == "band" else synth.random_mask(3, seed=logn)
    y = run_gpu(inp, mask)
    ref = oracle_full(inp, mask)
    check(y, ref, 1e-5)


def test_delta_filter_is_identity_times_gates():
    _say("delta filter")
    inp = synth.generate(2, 2, 4096, 1, "f32", gated=True, seed=3)
    inp.k = torch.ones_like(inp.k)
    y = run_gpu(inp)
    ref = inp.f64("v") * (inp.f64("u") * inp.f64("w"))
    check(y, ref, 1e-6)


def test_causality_on_gpu():
    _say("causality")
    inp = synth.generate(1, 2, 4096, 4096, "f32", gated=False, seed=4)
    y1 = run_gpu(inp)
    t0 = 3000
    inp.u[..., t0] += 100.0
    y2 = run_gpu(inp)
    scale = np.abs(y1).max()
    assert np.max(np.abs(y1[..., :t0] - y2[..., :t0])) < 1e-5 * scale
    assert np.max(np.abs(y1[..., t0:] - y2[..., t0:])) > 1.0


def test_deterministic_across_runs():
    _say("determinism")
    inp = synth.generate(4, 8, 16384, 16384, "bf16", gated=True, seed=6)
    assert np.array_equal(run_gpu(inp), run_gpu(inp))


@pytest.mark.parametrize("dtype,logn,L", [("f32", 10, 1024), ("f16", 12, 300), ("bf16", 14, 16384)])
def test_prepared_filter_matches_oracle_spectrum(dtype, logn, L):
    N = 1 << logn
    _say(f"export K_f dtype={dtype} N={N} L={L}")
    inp = synth.generate(1, 3, N, L, dtype, seed=8)
    k = inp.k.cuda()
    K_f = fc.alloc_filter(3, N, k.dtype)
    fc.fftconv_prepare_filter(k, N, K_f)
    got = fc.fftconv_export_filter_rfft(K_f, 3, N, k.dtype)
    k64 = inp.f64("k")
    for h in range(3):
        x = np.zeros(2 * N, complex)
        x[:L] = k64[h]
        want = oracle.fft(x)[:N + 1]
        tol = 1e-6 if dtype == "f32" else 2e-3
        assert np.linalg.norm(got[h] - want) / np.linalg.norm(want) < tol


# ---- N = 1024 in fp16 / bf16 storage runs on the matrix-core pair kernel
# (H >= 8: each XCD owns a channel range, ragged when 8 does not divide H)
@pytest.mark.parametrize("B,H", [(1, 1), (2, 1), (3, 5), (1, 7), (64, 3), (2, 8), (1, 9), (5, 13), (7, 50)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pair_kernel_batches(B, H, dtype):
    _say(f"pair kernel B={B} H={H} {dtype}")
    inp = synth.generate(B, H, 1024, 1024, dtype, gated=True, seed=B * 100 + H)
    y = run_gpu(inp)
    ref = oracle_full(inp)
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("gates", ["none", "w", "v"])
def test_pair_kernel_gates(gates):
    _say(f"pair kernel gates={gates}")
    inp = synth.generate(4, 3, 1024, 700, "f16", gated=True, seed=31)
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    y = run_gpu(inp)
    ref = oracle.direct(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL["f16"])


@pytest.mark.parametrize("kind", ["band", "random"])
def test_pair_kernel_mask(kind):
    _say(f"pair kernel mask {kind}")
    inp = synth.generate(3, 12, 1024, 1024, "f16", gated=True, seed=32)
    mask = synth.band_mask(12, 27) if kind == "band" else synth.random_mask(12, seed=3)
    y = run_gpu(inp, mask)
    ref = oracle_full(inp, mask)
    check(y, ref, TOL["f16"])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pair_layout_spectrum(dtype):
    _say(f"pair layout export {dtype}")
    N, L = 1024, 555
    inp = synth.generate(1, 3, N, L, dtype, seed=33)
    k = inp.k.cuda()
    K_f = fc.alloc_filter(3, N, k.dtype)
    fc.fftconv_prepare_filter(k, N, K_f)
    got = fc.fftconv_export_filter_rfft(K_f, 3, N, k.dtype)
    k64 = inp.f64("k")
    for h in range(3):
        x = np.zeros(2 * N, complex)
        x[:L] = k64[h]
        want = oracle.fft(x)[:N + 1]
        assert np.linalg.norm(got[h] - want) / np.linalg.norm(want) < 2e-3


# ---- N = 16384 in fp16 / bf16 storage runs on the three-stage matrix-core kernel
@pytest.mark.parametrize("gates,dtype,L", [("both", "bf16", 16384), ("none", "f16", 5000),
                                           ("w", "f16", 16384), ("v", "bf16", 1)])
def test_pair16k_gates_and_partial(gates, dtype, L):
    _say(f"pair16k gates={gates} {dtype} L={L}")
    inp = synth.generate(3, 2, 16384, L, dtype, gated=True, seed=41)
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("kind", ["band", "random"])
def test_pair16k_mask(kind):
    _say(f"pair16k mask {kind}")
    inp = synth.generate(2, 3, 16384, 16384, "f16", gated=True, seed=42)
    mask = synth.band_mask(3, 27) if kind == "band" else synth.random_mask(3, seed=7)
    y = run_gpu(inp, mask)
    ref = oracle_full(inp, mask)
    check(y, ref, TOL["f16"])


# ---- N = 2048, 4096, 8192 in fp16 / bf16 storage run on the same kernel with R = 4, 8, 16
# outer rows: 32 / R pairs of consecutive channels share a workgroup, so H not a multiple
# of 32 / R leaves a partial last group of channels
@pytest.mark.parametrize("logn", [11, 12, 13])
@pytest.mark.parametrize("B,H", [(1, 1), (2, 9), (4, 16), (5, 3), (1, 37)])
def test_pair_r_groups(logn, B, H):
    N = 1 << logn
    dtype = "f16" if (B + H) % 2 else "bf16"
    _say(f"pair R kernel N={N} B={B} H={H} {dtype}")
    inp = synth.generate(B, H, N, N, dtype, gated=True, seed=logn * 1000 + B * 100 + H)
    y = run_gpu(inp)
    ref = oracle_full(inp)
    check(y, ref, TOL[dtype])


@pytest.mark.parametrize("logn", [11, 12, 13])
@pytest.mark.parametrize("gates", ["none", "w", "v"])
def test_pair_r_gates_and_partial(logn, gates):
    N = 1 << logn
    _say(f"pair R kernel N={N} gates={gates}")
    inp = synth.generate(3, 7, N, N // 3, "f16", gated=True, seed=logn * 10 + len(gates))
    if gates in ("none", "v"):
        inp.w = None
    if gates in ("none", "w"):
        inp.v = None
    y = run_gpu(inp)
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(y, ref, TOL["f16"])


@pytest.mark.parametrize("logn", [11, 12, 13])
@pytest.mark.parametrize("kind", ["band", "random"])
def test_pair_r_mask(logn, kind):
    N = 1 << logn
    _say(f"pair R kernel N={N} mask {kind}")
    H = 11
    inp = synth.generate(2, H, N, N, "bf16", gated=True, seed=logn + 50)
    mask = synth.band_mask(H, 27) if kind == "band" else synth.random_mask(H, seed=logn)
    y = run_gpu(inp, mask)
    ref = oracle_full(inp, mask)
    check(y, ref, TOL["bf16"])


@pytest.mark.parametrize("logn", [11, 13])
def test_pair_r_layout_spectrum(logn):
    # the exported spectrum of the R-row layout matches the oracle's FFT of the taps
    N, L = 1 << logn, 777
    _say(f"pair R layout export N={N}")
    inp = synth.generate(1, 5, N, L, "f16", seed=logn + 60)
    k = inp.k.cuda()
    K_f = fc.alloc_filter(5, N, k.dtype)
    fc.fftconv_prepare_filter(k, N, K_f)
    got = fc.fftconv_export_filter_rfft(K_f, 5, N, k.dtype)
    k64 = inp.f64("k")
    for h in range(5):
        x = np.zeros(2 * N, complex)
        x[:L] = k64[h]
        want = oracle.fft(x)[:N + 1]
        assert np.linalg.norm(got[h] - want) / np.linalg.norm(want) < 2e-3
