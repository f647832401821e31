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
from parity import check

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
    # du, dw, dv per (b, h) sequence; dk per channel h (its rows)
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        if b is None:
            assert a is None, name
            continue
        check(a, b, tol, name)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gates", ["both", "none", "w", "v"])
def test_bwd_n1024(dtype, gates):
    B, H, N, L = 3, 2, 1024, 1024
    _say(f"bwd N={N} {dtype} gates={gates}")
    inp, dy = _case(B, H, N, L, dtype, gates, seed=71)
    got = _run(inp, dy)
    want = oracle.direct_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("dtype,N,L", [("f32", 2048, 2048), ("f16", 4096, 1000), ("bf16", 2048, 2048),
                                       ("f16", 8192, 8192), ("bf16", 16384, 16384),
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


@pytest.mark.parametrize("gates", ["w", "both", "none", "v"])
def test_bwd_n16384_channels(gates):
    # N = 16384: du and dw come from one kernel call, dk from the pairs' spectra of u w and
    # one correlation per pair; an odd batch (the last pair has one sequence), enough
    # channels for the per-XCD channel split, every combination of the gates
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


@pytest.mark.parametrize("kind", ["band", "random"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_mask_multipass_half(kind, dtype):
    # the three-pass path in half precision with a frequency mask (the row pass skips
    # the dropped tiles under the band mask), gated, an odd batch
    B, H, N = 3, 2, 1 << 17
    _say(f"bwd mask {kind} N={N} {dtype}")
    inp, dy = _case(B, H, N, 5000, dtype, "both", seed=N + 11)
    mask = synth.band_mask(H, 27) if kind == "band" else synth.random_mask(H, seed=N + 1)
    got = _run(inp, dy, mask)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"), mask)
    _check(got, want, TOL[dtype])


def test_bwd_n2_20():
    # N = 2^20 (the 1M workload's length): all four gradients of two whole channels
    B, H, N = 1, 2, 1 << 20
    _say(f"bwd N={N} f16 B={B} H={H}")
    inp, dy = _case(B, H, N, N, "f16", "both", seed=2020)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL["f16"])


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_n16384_batches(B, dtype):
    # N = 16384: one pair of batch rows per channel (B = 2), a lone row (B = 1) and two
    # pairs summed by the reduction (B = 4); a filter shorter than the sequence
    H, N, L = 5, 16384, 9000
    _say(f"bwd N={N} B={B} H={H} L={L} {dtype}")
    inp, dy = _case(B, H, N, L, dtype, "both", seed=900 + B)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("dtype,loc,dscale", [("bf16", 2.0, 1e3), ("f16", 4.0, 1.0), ("bf16", 0.0, 1e-3)])
def test_bwd_n16384_range(dtype, loc, dscale):
    # the filter gradient's per-pair spectrum scale: u, w ~ N(loc, 1) (a large zero bin),
    # and dy scaled far from unit size
    B, H, N = 2, 3, 16384
    _say(f"bwd range N={N} {dtype} loc={loc} dy x{dscale}")
    inp, dy = _case(B, H, N, N, dtype, "both", seed=1600 + int(loc))
    inp.u = (inp.u.double() + loc).to(inp.u.dtype)
    inp.w = (inp.w.double() + loc).to(inp.w.dtype)
    dy = (dy.double() * dscale).to(dy.dtype)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("N,H", [(2048, 3), (2048, 17), (4096, 5), (8192, 3)])
@pytest.mark.parametrize("gates", ["both", "none", "w", "v"])
def test_bwd_r_rows_groups(N, H, gates):
    # N = 2048 .. 8192 (fp16 / bf16): dk from the per-group spectra of u w (a workgroup
    # holds 2^(14 - log2 N) channels: 8, 4, 2) and one correlation per group; H not a
    # multiple of the group (a partial last group), an odd batch (a lone last row)
    B, L = 3, N - 100
    dtype = "bf16" if N == 4096 else "f16"
    _say(f"bwd N={N} B={B} H={H} gates={gates} {dtype}")
    inp, dy = _case(B, H, N, L, dtype, gates, seed=N + H)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


@pytest.mark.parametrize("N", [2048, 4096, 8192])
@pytest.mark.parametrize("B", [1, 4])
def test_bwd_r_rows_batches(N, B):
    # one lone row (B = 1) and two pairs summed by the reduction (B = 4), more channels
    # than one group
    H = 6
    _say(f"bwd N={N} B={B} H={H}")
    inp, dy = _case(B, H, N, N, "f16", "both", seed=7 * N + B)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL["f16"])


@pytest.mark.parametrize("N", [2048, 8192])
@pytest.mark.parametrize("kind", ["band", "random"])
def test_bwd_r_rows_mask(N, kind):
    # the correlation mode under a frequency mask (each channel of a group its own mask row)
    B, H = 2, 5
    _say(f"bwd mask {kind} N={N}")
    inp, dy = _case(B, H, N, N, "bf16", "both", seed=N + 3)
    mask = synth.band_mask(H, 27) if kind == "band" else synth.random_mask(H, seed=N + 5)
    got = _run(inp, dy, mask)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"), mask)
    _check(got, want, TOL["bf16"])


@pytest.mark.parametrize("N,dtype,loc,dscale", [(2048, "bf16", 2.0, 1e3), (8192, "f16", 4.0, 1.0),
                                                (4096, "bf16", 0.0, 1e-3)])
def test_bwd_r_rows_range(N, dtype, loc, dscale):
    # one spectrum scale per group: u, w ~ N(loc, 1) and dy far from unit size, with one
    # channel of the group much smaller than the others
    B, H = 2, 4
    _say(f"bwd range N={N} {dtype} loc={loc} dy x{dscale}")
    inp, dy = _case(B, H, N, N, dtype, "both", seed=N + int(loc))
    u = inp.u.double() + loc
    u[:, 1] *= 1e-2
    inp.u = u.to(inp.u.dtype)
    inp.w = (inp.w.double() + loc).to(inp.w.dtype)
    dy = (dy.double() * dscale).to(dy.dtype)
    got = _run(inp, dy)
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"))
    _check(got, want, TOL[dtype])


def test_bwd_gated_bf16_n16k_full_size():
    # the N = 16384 benchmark configuration (gated_bf16_n16k: B = 4, H = 2560, bf16) run
    # whole; every gradient of 12 channels spread over the range (all their batch rows,
    # their dk rows) compared with the oracle run on those channels alone
    wl = synth.WORKLOADS["gated_bf16_n16k"]
    _say(f"bwd {wl.name} full size")
    inp = synth.generate_workload(wl.name)
    g = torch.Generator().manual_seed(4243)
    dy = torch.randn(inp.u.shape, generator=g, dtype=torch.float32).to(inp.u.dtype)
    got = _run(inp, dy)
    hs = np.array([0, 1, 7, 255, 256, 1023, 1280, 1281, 2047, 2300, 2558, 2559])
    sub = lambda t: t[:, hs]
    want = oracle.fft_bwd(sub(inp.f64("u")), inp.f64("k")[hs], sub(dy.double().numpy()), sub(inp.f64("w")),
                          sub(inp.f64("v")))
    for name, a, b in zip(("du", "dk", "dw", "dv"), got, want):
        check(a[hs] if name == "dk" else a[:, hs], b, TOL["bf16"], f"{name} channels {list(hs)}")


@pytest.mark.parametrize("dtype,N,B,H,masked", [("f16", 1024, 3, 6, False), ("bf16", 16384, 3, 5, False),
                                                ("bf16", 16384, 2, 3, True), ("f16", 8192, 2, 5, False)])
def test_bwd_gradient_subsets(dtype, N, B, H, masked):
    # each gradient asked for alone, and dv with dk, du with dw: the call takes other routes
    # then (dv from the forward call instead of the dk chain's first pass at N = 16384, du or
    # dw alone from the forward call on a conjugated copy of the spectrum, dk alone from the
    # spectrum-only pass); every result is checked against the oracle
    L = N - 37
    _say(f"bwd subsets {dtype} N={N} B={B} H={H} masked={masked}")
    inp, dy = _case(B, H, N, L, dtype, "both", 71)
    mask = None
    if masked:   # a band on every channel, a random mask on the second
        mask = synth.band_mask(H, 27)
        mask[1] = synth.random_mask(H, seed=N + 9)[1]
    want = oracle.fft_bwd(inp.f64("u"), inp.f64("k"), dy.double().numpy(), inp.f64("w"), inp.f64("v"), mask)
    dev = torch.device("cuda")
    u, k, w, v, g = (t.to(dev) for t in (inp.u, inp.k, inp.w, inp.v, dy))
    m = None if mask is None else torch.from_numpy(mask).to(dev)
    K_f = fc.alloc_filter(H, N, u.dtype, dev)
    fc.fftconv_prepare_filter(k, N, K_f, fc.alloc_workspace(1, H, N, u.dtype, dev))
    ws = torch.empty(fc.fftconv_bwd_workspace_bytes(B, H, N, u.dtype), dtype=torch.uint8, device=dev)
    names = ("du", "dk", "dw", "dv")
    for subset in (("du",), ("dw",), ("dv",), ("dk",), ("dv", "dk"), ("du", "dw")):
        outs = {n: (torch.empty((H, L), dtype=u.dtype, device=dev) if n == "dk" else torch.empty_like(u))
                for n in subset}
        fc.fftconv_bwd(g, u, K_f, w, v, outs.get("du"), outs.get("dk"), outs.get("dw"), outs.get("dv"), L, m, ws)
        torch.cuda.synchronize()
        for n in subset:
            check(outs[n].float().cpu().double().numpy(), want[names.index(n)], TOL[dtype], f"{n} of {subset}")
