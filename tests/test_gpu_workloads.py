"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the oracle sequence by sequence.

The five workloads (long_fft_convolution_amd.synth.WORKLOADS) run whole on the
GPU.  The oracle then recomputes
  - every sequence where its FFT route finishes in seconds (the 1024- and
    16384-point workloads: 4, 49,152 and 10,240 sequences), or
  - a seeded set of whole sequences, the first and last included (the 1M and
    4M-point workloads: its FFT route takes seconds per sequence there),
    plus the exact definition at seeded sample positions spread over every
    sequence (the direct sum for dense filters, the circular form with the
    masked filter for the frequency-sparse one).
Each comparison goes through tests/parity.check: whole relL2, the worst
per-sequence relL2 and the max-abs error are printed ([parity] lines) and the
first two are held to the workload's tolerance.
"""
import concurrent.futures
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


def _sample_points(wl, n, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, wl.B, n)
    h = rng.integers(0, wl.H, n)
    t = rng.integers(0, wl.N, n)
    edge = np.array([[0, 0, 0], [wl.B - 1, wl.H - 1, wl.N - 1], [0, wl.H - 1, 1],
                     [wl.B - 1, 0, wl.N - 2], [0, 0, min(wl.L, wl.N - 1)]])
    return np.concatenate([np.stack([b, h, t], 1), edge]).astype(np.int64)


def _run_full(inp, wl):
    dev = torch.device("cuda")
    u = inp.u.to(dev)
    k = inp.k.to(dev)
    w = None if inp.w is None else inp.w.to(dev)
    v = None if inp.v is None else inp.v.to(dev)
    mask = None if inp.mask is None else torch.from_numpy(inp.mask).to(dev)
    K_f = fc.alloc_filter(wl.H, wl.N, u.dtype, dev)
    fc.fftconv_prepare_filter(k, wl.N, K_f, fc.alloc_workspace(1, wl.H, wl.N, u.dtype, dev))
    out = torch.empty_like(u)
    fc.fftconv_fwd(u, K_f, w, v, out, wl.L, mask, fc.alloc_workspace(wl.B, wl.H, wl.N, u.dtype, dev))
    torch.cuda.synchronize()
    return out


def _sequences(inp, wl, seqs):
    """Oracle (route F) for the given flat sequence indices b * H + h, each as its own channel."""
    b = torch.from_numpy(seqs // wl.H)
    h = torch.from_numpy(seqs % wl.H)
    g = lambda t: None if t is None else t[b, h].to(torch.float64).numpy()[None]
    mask = None if inp.mask is None else inp.mask[h.numpy()]
    return oracle.fft_conv(g(inp.u), inp.k[h].to(torch.float64).numpy(), g(inp.w), g(inp.v), mask=mask)[0]


@pytest.mark.parametrize("name", ["ungated_fp32_n1k", "gated_fp16_n1k", "gated_bf16_n16k"])
def test_on_chip_workload_every_sequence(name):
    wl = synth.WORKLOADS[name]
    _say(f"workload {name}: every sequence")
    inp = synth.generate_workload(name)
    out = _run_full(inp, wl)
    got = out.double().cpu().numpy()
    del out
    ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"))
    check(got, ref, TOL[wl.dtype], f"{name} (all {wl.B * wl.H} sequences)")
    if wl.N <= 1024:
        # the direct sums agree with route F on this size; compare them too
        pts = _sample_points(wl, 256, seed=1)
        ref_d = oracle.direct_points(inp.f64("u"), inp.f64("k"), pts, inp.f64("w"), inp.f64("v"))
        check(got[pts[:, 0], pts[:, 1], pts[:, 2]], ref_d, TOL[wl.dtype], f"{name} (direct sums at samples)")


@pytest.mark.parametrize("name,nseq", [("ungated_fp16_n1m", 16), ("partial_sparse_n4m", 4)])
def test_long_workload_sequences_and_samples(name, nseq):
    wl = synth.WORKLOADS[name]
    _say(f"workload {name}: {nseq} whole sequences and samples")
    inp = synth.generate_workload(name)
    out = _run_full(inp, wl)
    assert torch.isfinite(out).all()
    S = wl.B * wl.H
    rng = np.random.default_rng(3)
    seqs = np.concatenate([[0, S - 1], rng.choice(np.arange(1, S - 1), nseq - 2, replace=False)])
    got = out.view(S, wl.N)[torch.from_numpy(seqs).cuda()].double().cpu().numpy()
    check(got, _sequences(inp, wl, seqs), TOL[wl.dtype], f"{name} ({nseq} whole sequences)")
    # samples spread over the sequences: every sequence for a dense filter (the direct
    # sum costs O(t) per output); for the masked one 16 channels, since each needs its
    # masked filter through two 2N-point FFTs (run in parallel threads)
    pts = _sample_points(wl, 64, seed=1)
    if inp.mask is not None:
        hs = np.concatenate([[0, wl.H - 1], rng.choice(np.arange(1, wl.H - 1), 14, replace=False)])
        pts[:64, 1] = hs[np.arange(64) % 16]
    gotp = out[pts[:, 0], pts[:, 1], pts[:, 2]].double().cpu().numpy()
    ref = np.empty(len(pts))
    keys = np.unique(pts[:, 0] * wl.H + pts[:, 1])

    def one(s):
        b, h = divmod(int(s), wl.H)
        sel = (pts[:, 0] == b) & (pts[:, 1] == h)
        if inp.mask is None:
            f64 = lambda t: None if t is None else t[b:b + 1, h:h + 1].to(torch.float64).numpy()
            q = np.stack([np.zeros(sel.sum(), np.int64), np.zeros(sel.sum(), np.int64), pts[sel, 2]], 1)
            ref[sel] = oracle.direct_points(f64(inp.u), inp.k[h:h + 1].to(torch.float64).numpy(), q,
                                            f64(inp.w), f64(inp.v))
        else:
            kp = oracle.masked_filter(inp.k[h].to(torch.float64).numpy(), wl.N, inp.mask[h])
            ref[sel] = oracle.circular_points(inp.u[b, h].to(torch.float64).numpy(), kp, pts[sel, 2])

    with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(one, keys))
    check(gotp, ref, TOL[wl.dtype], f"{name} (samples over {len(keys)} sequences)")
