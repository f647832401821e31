"""The forward call captured into a HIP graph (torch.cuda.CUDAGraph) after the
filter is prepared: the prepare built the library's constant tables, so the
captured call neither allocates nor synchronises.  The graph is replayed
several times with eager GPU work and synchronisations between replays (new
inputs copied into the captured buffers each time); every replay is compared
with the oracle and with the same call run eagerly."""
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


@pytest.mark.parametrize("dtype,B,H,N,L,masked", [
    ("f16", 4, 9, 1024, 1024, False),        # N = 1024 matrix-core kernel
    ("bf16", 3, 4, 16384, 16384, True),      # N = 16384 matrix-core kernel, mask
    ("f32", 2, 3, 4096, 4096, False),        # fused fp32 kernel
    ("f16", 1, 3, 1 << 17, 5000, True),      # three-pass path with its workspace, mask
])
def test_forward_in_graph(dtype, B, H, N, L, masked):
    _say(f"graph {dtype} B={B} H={H} N={N} L={L} masked={masked}")
    dev = torch.device("cuda")
    first = synth.generate(B, H, N, L, dtype, gated=True, seed=N + 1)
    k = first.k.to(dev)
    mask_np = synth.random_mask(H, seed=N) if masked else None
    mask = None if mask_np is None else torch.from_numpy(mask_np).to(dev)
    K_f = fc.alloc_filter(H, N, k.dtype, dev)
    fc.fftconv_prepare_filter(k, N, K_f, fc.alloc_workspace(1, H, N, k.dtype, dev))
    u = torch.empty(first.u.shape, dtype=k.dtype, device=dev)
    w = torch.empty_like(u)
    v = torch.empty_like(u)
    out = torch.empty_like(u)
    ws = fc.alloc_workspace(B, H, N, k.dtype, dev)
    for t, src in ((u, first.u), (w, first.w), (v, first.v)):
        t.copy_(src)
    # warm-up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fc.fftconv_fwd(u, K_f, w, v, out, L, mask, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fc.fftconv_fwd(u, K_f, w, v, out, L, mask, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        inp = first if rep == 0 else synth.generate(B, H, N, L, dtype, gated=True, seed=N + 1 + rep)
        inp.k = first.k   # the captured call reads the prepared filter
        for t, src in ((u, inp.u), (w, inp.w), (v, inp.v)):
            t.copy_(src)
        junk = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        eager = torch.empty_like(out)
        fc.fftconv_fwd(u, K_f, w, v, eager, L, mask, ws)
        torch.cuda.synchronize()
        assert torch.equal(eager, out), f"replay {rep} differs from the eager call"
        ref = oracle.fft_conv(inp.f64("u"), inp.f64("k"), inp.f64("w"), inp.f64("v"), mask=mask_np)
        check(got, ref, TOL[dtype], f"replay {rep}")
        del junk
