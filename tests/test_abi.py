"""C-ABI checks that need no GPU: the library loads, exports every function
include/fftconv.h declares, computes its size helpers, and rejects bad
arguments before it would touch the device (every case below fails
validation, so nothing is launched).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fftconv.h")

fc = pytest.importorskip("long_fft_convolution_amd")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fftconv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["fftconv_prepare_filter", "fftconv_fwd", "fftconv_filter_bytes",
              "fftconv_workspace_bytes", "fftconv_mask_blocks", "fftconv_status_string",
              "fftconv_last_error", "fftconv_export_filter_rfft"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fc.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert hasattr(fc, name), f"binding lacks {name}"


def test_size_helpers():
    F32, F16, BF16 = fc.FFTCONV_F32, fc.FFTCONV_F16, fc.FFTCONV_BF16
    # header 256 B + scales rounded to 256 B + H*N bins of 8 B (fp32) or 4 B (fp16);
    # the matrix-core kernel for N = 1024 (fp16/bf16) keeps all 2N bins of the spectrum;
    # the one for N = 2048 .. 16384 keeps rows f_c = 0 .. R/2 of the R x 1024 bin grid,
    # R = 2N / 1024 (at N = 16384: 17 * 1024 bins)
    assert fc.fftconv_filter_bytes(4, 1024, F32) == 256 + 256 + 4 * 1024 * 8
    assert fc.fftconv_filter_bytes(768, 1024, F16) == 256 + 3072 + 768 * 2048 * 4
    assert fc.fftconv_filter_bytes(768, 2048, F16) == 256 + 3072 + 768 * 3 * 1024 * 4   # rows f mod 4 in [0, 2]
    assert fc.fftconv_filter_bytes(768, 8192, BF16) == 256 + 3072 + 768 * 9 * 1024 * 4  # rows f mod 16 in [0, 8]
    assert fc.fftconv_filter_bytes(2560, 16384, BF16) == 256 + 10240 + 2560 * 17 * 1024 * 4
    assert fc.fftconv_filter_bytes(2560, 16384, F32) == 256 + 10240 + 2560 * 16384 * 8
    assert fc.fftconv_filter_bytes(0, 1024, F32) == 0
    assert fc.fftconv_filter_bytes(4, 1000, F32) == 0
    assert fc.fftconv_filter_bytes(4, 1 << 23, F32) == 0
    assert fc.fftconv_filter_bytes(4, 1024, 7) == 0
    for n in (1024, 16384):
        assert fc.fftconv_workspace_bytes(64, 768, n, F16) == 0
    # multi-pass workspace per sequence of a chunk: one complex value per point
    # in the storage type plus 2 * 8192 fp32 complex values; the intermediate
    # of a chunk takes 128 MiB
    extra = 2 * 8192 * 8
    ws = fc.fftconv_workspace_bytes(1, 256, 1 << 20, F16)
    assert ws == 32 * ((1 << 20) * 4 + extra)
    assert fc.fftconv_workspace_bytes(1, 1, 1 << 20, F16) == (1 << 20) * 4 + extra
    assert fc.fftconv_workspace_bytes(1, 1, 1 << 20, F32) == (1 << 20) * 8 + extra
    assert fc.fftconv_workspace_bytes(1, 256, 1 << 20, F32) == 16 * ((1 << 20) * 8 + extra)
    assert fc.fftconv_mask_blocks(1 << 22) == 128
    assert fc.fftconv_mask_blocks(1024) == 128
    assert fc.fftconv_mask_blocks(512) == 0
    assert fc.fftconv_status_string(0) == "ok"
    assert "workspace" in fc.fftconv_status_string(3)


def _fwd(**kw):
    lib = fc.lib()
    a = dict(u=0x10000, K_f=0x20000, w=None, v=None, out=0x30000, B=1, H=1, N=1024, L=1024,
             mask=None, dtype=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.fftconv_fwd(a["u"], a["K_f"], a["w"], a["v"], a["out"], a["B"], a["H"], a["N"],
                           a["L"], a["mask"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,text", [
    (dict(N=1000), 2, "power of two"),
    (dict(N=512), 2, "power of two"),
    (dict(N=1 << 23), 2, "power of two"),
    (dict(dtype=9), 2, "dtype"),
    (dict(L=0), 1, "L_filter"),
    (dict(L=2048), 1, "L_filter"),
    (dict(B=-1), 1, ">= 0"),
    (dict(u=None), 1, "non-null"),
    (dict(out=None), 1, "non-null"),
    (dict(K_f=None), 1, "non-null"),
    (dict(u=0x10004), 1, "aligned"),
    (dict(w=0x40008), 1, "aligned"),
    (dict(out=0x10000 + 16), 1, "overlaps"),
    (dict(N=1 << 20, L=1 << 20, out=0x10000000 * 4), 3, "workspace"),
])
def test_fwd_validation(kw, status, text):
    assert _fwd(**kw) == status
    assert text in fc.fftconv_last_error()


def test_fwd_empty_batch_is_a_no_op():
    assert _fwd(B=0, u=None, out=None, K_f=None) == 0
    assert _fwd(H=0) == 0


def test_prepare_validation():
    lib = fc.lib()
    good = dict(k=0x10000, H=2, L=100, N=1024, dt=0, K_f=0x100000, kb=1 << 20, ws=None, wsb=0)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return lib.fftconv_prepare_filter(a["k"], a["H"], a["L"], a["N"], a["dt"], a["K_f"],
                                          a["kb"], a["ws"], a["wsb"], None)

    assert call(H=0) == 1
    assert call(L=2000) == 1
    assert call(N=3000) == 2
    assert call(kb=100) == 1 and "needs" in fc.fftconv_last_error()
    assert call(k=None) == 1
    assert call(k=0x10002) == 1
    assert call(K_f=0x10000 + 256) == 1 and "overlaps" in fc.fftconv_last_error()
    assert call(N=1 << 20, L=5, kb=1 << 30) == 3


def test_bwd_workspace_bytes():
    F16, BF16, F32 = fc.FFTCONV_F16, fc.FFTCONV_BF16, fc.FFTCONV_F32
    # fp32: conjugated K_f + u*w + the B*H sequence spectra + correlations + mask rows
    # + the forward workspace, each region rounded up to 256 bytes
    B, H, N = 2, 3, 2048

    def up(x):
        return (x + 255) // 256 * 256

    S = B * H
    want = (up(fc.fftconv_filter_bytes(H, N, F32)) + up(S * N * 4) + up(fc.fftconv_filter_bytes(S, N, F32))
            + up(S * N * 4) + up(S * 128) + up(fc.fftconv_workspace_bytes(1, S, N, F32)))
    assert fc.fftconv_bwd_workspace_bytes(B, H, N, F32) == want
    # N = 2048 .. 8192 in fp16 / bf16: the conjugated K_f, then per group (the 2^(14 - log2 N)
    # channels of one workgroup, of one pair of batch rows) a 32-row spectrum and one scale
    # per channel, and one correlation row per pair of batch rows and channel
    for Nq, Pch in ((2048, 8), (4096, 4), (8192, 2)):
        for Bq, Hq in ((1, 3), (3, 9), (4, 16)):
            PB = (Bq + 1) // 2
            G = (Hq + Pch - 1) // Pch * PB
            want = (up(fc.fftconv_filter_bytes(Hq, Nq, F16)) + up(G * 32 * 1024 * 4) + up(G * Pch * 4)
                    + up(PB * Hq * Nq * 2))
            assert fc.fftconv_bwd_workspace_bytes(Bq, Hq, Nq, F16) == want, (Nq, Bq, Hq)
    # N = 1024 in fp16 / bf16: only the conjugated K_f (the gradients come from kernels
    # that need no other scratch); fp32 keeps the whole layout
    for dt in (F16, BF16):
        assert fc.fftconv_bwd_workspace_bytes(B, H, 1024, dt) == up(fc.fftconv_filter_bytes(H, 1024, dt))
    # N = 16384 in fp16 / bf16: the conjugated K_f, then per pair of batch rows its
    # spectrum of u*w (32 rows x 1024 bins x fp16 re/im), its scale and its correlation
    for Bq in (1, 2, 3):
        P = H * ((Bq + 1) // 2)
        want = (up(fc.fftconv_filter_bytes(H, 16384, BF16)) + up(P * 32 * 1024 * 4) + up(P * 4)
                + up(P * 16384 * 2))
        assert fc.fftconv_bwd_workspace_bytes(Bq, H, 16384, BF16) == want
    assert fc.fftconv_bwd_workspace_bytes(B, H, 1024, F32) > up(fc.fftconv_filter_bytes(H, 1024, F32)) + B * H * 1024 * 4
    assert fc.fftconv_bwd_workspace_bytes(B, H, 1 << 20, F32) > 0
    assert fc.fftconv_bwd_workspace_bytes(B, H, 1000, F16) == 0
    assert fc.fftconv_bwd_workspace_bytes(B, 0, N, F16) == 0


def test_bwd_validation():
    lib = fc.lib()
    N = 1024
    good = dict(dy=0x10000, u=0x20000, K_f=0x30000, w=0x40000, v=0x50000, du=0x60000, dk=0x70000,
                dw=0x80000, dv=0x90000, B=1, H=2, N=N, L=N, m=None, dt=0, ws=0x1000000, wsb=1 << 40)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return lib.fftconv_bwd(a["dy"], a["u"], a["K_f"], a["w"], a["v"], a["du"], a["dk"], a["dw"], a["dv"],
                               a["B"], a["H"], a["N"], a["L"], a["m"], a["dt"], a["ws"], a["wsb"], None)

    assert call(dt=7) == 2
    assert call(N=1000) == 2
    assert call(L=0) == 1
    assert call(B=-1) == 1
    assert call(H=0) == 0
    assert call(w=None) == 1 and "dw needs" in fc.fftconv_last_error()
    assert call(v=None) == 1 and "dv needs" in fc.fftconv_last_error()
    assert call(dy=None) == 1
    assert call(du=0x60004) == 1 and "aligned" in fc.fftconv_last_error()
    assert call(du=0x20000 + 256) == 1 and "overlaps" in fc.fftconv_last_error()
    assert call(ws=None) == 3
    assert call(wsb=16) == 3


def test_short_filter_abi():
    lib = fc.lib()
    F16, F32 = fc.FFTCONV_F16, fc.FFTCONV_F32
    # the 2048-point spectrum of the window: header, scales, 2048 bins of 4 bytes per channel
    assert fc.fftconv_short_filter_bytes(3, F16) == fc.fftconv_filter_bytes(3, 1024, F16)
    assert fc.fftconv_short_filter_bytes(3, F32) == 0

    def prep(**kw):
        a = dict(k=0x10000, H=2, L=100, dt=F16, K=0x100000, kb=1 << 20)
        a.update(kw)
        return lib.fftconv_prepare_short_filter(a["k"], a["H"], a["L"], a["dt"], a["K"], a["kb"], None)

    assert prep(dt=F32) == 2
    assert prep(L=1025) == 1 and "L_filter" in fc.fftconv_last_error()
    assert prep(L=0) == 1
    assert prep(kb=16) == 1

    def fwd(**kw):
        a = dict(u=0x10000, K=0x20000, w=None, v=None, out=0x30000, B=1, H=1, N=2048, L=100, dt=F16)
        a.update(kw)
        return lib.fftconv_fwd_short(a["u"], a["K"], a["w"], a["v"], a["out"], a["B"], a["H"], a["N"],
                                     a["L"], a["dt"], None)

    assert fwd(dt=F32) == 2
    assert fwd(N=1000) == 2 and "multiple of 1024" in fc.fftconv_last_error()
    assert fwd(N=512) == 2
    assert fwd(L=1025) == 1
    assert fwd(B=-1) == 1
    assert fwd(u=None) == 1
    assert fwd(out=0x30008) == 1 and "aligned" in fc.fftconv_last_error()
    assert fwd(out=0x10000 + 16) == 1 and "overlaps" in fc.fftconv_last_error()
    assert fwd(B=0, u=None, out=None, K=None) == 0


def test_short_bwd_validation():
    lib = fc.lib()
    F16, F32 = fc.FFTCONV_F16, fc.FFTCONV_F32
    good = dict(dy=0x10000, u=0x20000, K=0x30000, w=0x40000, v=0x50000, du=0x60000, dk=0x70000,
                dw=0x80000, dv=0x90000, B=1, H=2, N=2048, L=100, dt=F16)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return lib.fftconv_bwd_short(a["dy"], a["u"], a["K"], a["w"], a["v"], a["du"], a["dk"], a["dw"],
                                     a["dv"], a["B"], a["H"], a["N"], a["L"], a["dt"], None)

    assert call(dt=F32) == 2
    assert call(N=1000) == 2 and "multiple of 1024" in fc.fftconv_last_error()
    assert call(L=1025) == 1 and "L_filter" in fc.fftconv_last_error()
    assert call(L=0) == 1
    assert call(B=-1) == 1
    assert call(H=0) == 0
    assert call(w=None) == 1 and "dw needs" in fc.fftconv_last_error()
    assert call(v=None) == 1 and "dv needs" in fc.fftconv_last_error()
    assert call(dy=None) == 1
    assert call(K=None) == 1
    assert call(du=0x60008) == 1 and "aligned" in fc.fftconv_last_error()
    assert call(du=0x20000 + 256) == 1 and "overlaps" in fc.fftconv_last_error()
    assert call(dk=0x30000 + 16) == 1 and "overlaps" in fc.fftconv_last_error()
    # nothing asked for and no rows: nothing to do
    assert call(B=0, dy=None, u=None, du=None, dk=None, dw=None, dv=None) == 0


def test_eqlinear_abi():
    lib = fc.lib()
    F16, F32 = fc.FFTCONV_F16, fc.FFTCONV_F32
    # T/2 + 1 frequencies, two planes each: fp16 for half-precision storage, fp32 for fp32
    assert fc.fftconv_eqlinear_weight_bytes(8, 64, 32, F16) == 5 * 2 * 64 * 32 * 2
    assert fc.fftconv_eqlinear_weight_bytes(8, 64, 32, fc.FFTCONV_BF16) == 5 * 2 * 64 * 32 * 2
    assert fc.fftconv_eqlinear_weight_bytes(8, 64, 32, F32) == 5 * 2 * 64 * 32 * 4
    assert fc.fftconv_eqlinear_weight_bytes(6, 64, 32, F16) == 0
    assert fc.fftconv_eqlinear_weight_bytes(8, 64, 32, 7) == 0

    def prep(**kw):
        a = dict(W=0x10000, T=8, Co=64, Ci=32, dt=F16, Wf=0x100000, b=1 << 20)
        a.update(kw)
        return lib.fftconv_eqlinear_prepare(a["W"], a["T"], a["Co"], a["Ci"], a["dt"], a["Wf"], a["b"], None)

    assert prep(dt=7) == 2
    # fp32 weights need twice the fp16 bytes: a buffer sized for fp16 is rejected
    assert prep(dt=F32, b=5 * 2 * 64 * 32 * 2) == 1 and "needs" in fc.fftconv_last_error()
    assert prep(T=6) == 2 and "4, 8 or 16" in fc.fftconv_last_error()
    assert prep(Ci=48) == 2
    assert prep(Co=16) == 2
    assert prep(b=100) == 1
    assert prep(W=None) == 1

    def fwd(**kw):
        a = dict(x=0x10000, Wf=0x200000, y=0x400000, N=10, T=8, Ci=32, Co=64, dt=F16)
        a.update(kw)
        return lib.fftconv_eqlinear_fwd(a["x"], a["Wf"], a["y"], a["N"], a["T"], a["Ci"], a["Co"], a["dt"], None)

    assert fwd(T=12) == 2
    assert fwd(dt=7) == 2
    assert fwd(N=-1) == 1
    assert fwd(N=0, x=None, y=None) == 0
    assert fwd(y=0x400008) == 1 and "aligned" in fc.fftconv_last_error()
    assert fwd(y=0x10000 + 64) == 1 and "overlaps" in fc.fftconv_last_error()


def test_fwd_taps_abi():
    # forward from time-domain taps: the workspace holds the spectrum and the scratch;
    # every rejection below happens before anything is enqueued
    lib = fc.lib()
    F16 = fc.FFTCONV_F16
    H, N = 3, 1 << 20
    kf = (fc.fftconv_filter_bytes(H, N, F16) + 255) // 256 * 256
    need = fc.fftconv_fwd_taps_workspace_bytes(2, H, N, F16)
    assert need == kf + max(fc.fftconv_workspace_bytes(1, H, N, F16), fc.fftconv_workspace_bytes(2, H, N, F16))
    assert fc.fftconv_fwd_taps_workspace_bytes(2, H, 1024, F16) == (fc.fftconv_filter_bytes(H, 1024, F16) + 255) // 256 * 256
    assert fc.fftconv_fwd_taps_workspace_bytes(2, H, 1000, F16) == 0
    assert fc.fftconv_fwd_taps_workspace_bytes(-1, H, N, F16) == 0
    assert fc.fftconv_fwd_taps_workspace_bytes(2, 0, N, F16) == 0
    good = dict(u=0x100000, k=0x200000, w=None, v=None, out=0x40000000, B=2, H=H, N=N, L=1000, m=None,
                dt=F16, ws=0x80000000, wsb=need)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return lib.fftconv_fwd_taps(a["u"], a["k"], a["w"], a["v"], a["out"], a["B"], a["H"], a["N"], a["L"],
                                    a["m"], a["dt"], a["ws"], a["wsb"], None)

    assert call(dt=7) == 2
    assert call(N=1000) == 2
    assert call(L=0) == 1 and call(L=N + 1) == 1
    assert call(B=-1) == 1
    assert call(B=0) == 0 and call(H=0) == 0
    assert call(k=None) == 1
    assert call(ws=None) == 3 and call(wsb=need - 1) == 3
    assert call(ws=0x80000004) == 1 and "aligned" in fc.fftconv_last_error()
    assert call(k=0x80000000 + 4096) == 1 and "overlaps" in fc.fftconv_last_error()
    assert call(out=0x200000 + 64) == 1 and "overlaps" in fc.fftconv_last_error()
    # the forward call's own checks also run before the prepare is enqueued
    assert call(u=0x100004) == 1 and "aligned" in fc.fftconv_last_error()
    assert call(u=None) == 1
