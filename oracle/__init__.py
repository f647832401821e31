"""CPU oracle for the exact causal long FFT convolution (float64).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  The HIP library never
imports, links or calls anything here, and this module imports nothing from
the HIP package.

What is computed (FlashFFTConv summary page: "Summary" and "Key results" say
the method computes exact FFT convolutions; the "Measured effects" row on
fusing gating gives the gated form; "Approach" names partial and
frequency-sparse filters):

    y[b,h,t] = v[b,h,t] * sum_{s<=min(t,L-1)} k[h,s] * (u*w)[b,h,t-s],  t < N

Route D (``direct``) writes that sum out; route F (``fft_conv``) uses the
convolution theorem with the oracle's own radix-2 FFT (``fft``), which is the
only route that can apply a frequency mask (``oracle_fft_conv`` in the C file
states the mask reading).  Every function is pinned by the ``-m "not gpu"``
tests to brute force, closed forms or an independent library routine.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fftconv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C file with gcc (plain -O2, OpenMP, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-std=c11", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    lib.oracle_fft.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int]
    lib.oracle_fft.restype = ctypes.c_int
    lib.oracle_direct.argtypes = [_dp, _dp, _dp, _dp] + [ctypes.c_int64] * 4 + [_dp, ctypes.c_int]
    lib.oracle_direct.restype = ctypes.c_int
    lib.oracle_direct_points.argtypes = ([_dp, _dp, _dp, _dp] + [ctypes.c_int64] * 4
                                         + [_i64p, ctypes.c_int64, _dp, ctypes.c_int])
    lib.oracle_direct_points.restype = ctypes.c_int
    lib.oracle_fft_conv.argtypes = ([_dp, _dp, _dp, _dp] + [ctypes.c_int64] * 4
                                    + [_u8p, ctypes.c_int64, _dp, _dp, ctypes.c_int])
    lib.oracle_fft_conv.restype = ctypes.c_int
    lib.oracle_masked_filter.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _u8p, _dp]
    lib.oracle_masked_filter.restype = ctypes.c_int
    lib.oracle_circular_points.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, _i64p,
                                           ctypes.c_int64, _dp]
    lib.oracle_circular_points.restype = ctypes.c_int
    lib.oracle_mask_blocks.argtypes = [ctypes.c_int64]
    lib.oracle_mask_blocks.restype = ctypes.c_int64
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it only when no library exists)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=_dp):
    return None if a is None else a.ctypes.data_as(typ)


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()


def mask_blocks(N: int) -> int:
    return int(load().oracle_mask_blocks(N))


def fft(x, sign: int = -1, lib=None):
    """Complex FFT of length M (power of two); sign=-1 forward, +1 unnormalised inverse."""
    lib = lib or load()
    x = np.asarray(x, dtype=np.complex128)
    re = np.ascontiguousarray(x.real.copy())
    im = np.ascontiguousarray(x.imag.copy())
    rc = lib.oracle_fft(_ptr(re), _ptr(im), x.size, sign)
    if rc:
        raise ValueError("oracle_fft: length must be a power of two")
    return re + 1j * im


def direct(u, k, w=None, v=None, L=None, threads: int = 0, lib=None):
    """Route D over whole tensors: u, w, v (B, H, N); k (H, L)."""
    lib = lib or load()
    u, w, v, k = _f64(u), _f64(w), _f64(v), _f64(k)
    B, H, N = u.shape
    L = k.shape[1] if L is None else L
    y = np.empty((B, H, N), dtype=np.float64)
    rc = lib.oracle_direct(_ptr(u), _ptr(w), _ptr(v), _ptr(k), B, H, N, L, _ptr(y), threads)
    if rc:
        raise ValueError("oracle_direct: bad arguments")
    return y


def direct_points(u, k, pts, w=None, v=None, threads: int = 0, lib=None):
    """Route D at sampled (b, h, t) triples (pts: (P, 3) int64)."""
    lib = lib or load()
    u, w, v, k = _f64(u), _f64(w), _f64(v), _f64(k)
    B, H, N = u.shape
    L = k.shape[1]
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    out = np.empty(pts.shape[0], dtype=np.float64)
    rc = lib.oracle_direct_points(_ptr(u), _ptr(w), _ptr(v), _ptr(k), B, H, N, L,
                                  _ptr(pts, _i64p), pts.shape[0], _ptr(out), threads)
    if rc:
        raise ValueError("oracle_direct_points: bad arguments")
    return out


def fft_conv(u, k, w=None, v=None, mask=None, M=None, threads: int = 0, lib=None,
             return_imag: bool = False):
    """Route F over whole tensors, FFT size M (default 2N), optional (H, 128) mask."""
    lib = lib or load()
    u, w, v, k = _f64(u), _f64(w), _f64(v), _f64(k)
    B, H, N = u.shape
    L = k.shape[1]
    M = 2 * N if M is None else M
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    y = np.empty((B, H, N), dtype=np.float64)
    imag = ctypes.c_double(0.0)
    rc = lib.oracle_fft_conv(_ptr(u), _ptr(w), _ptr(v), _ptr(k), B, H, N, L,
                             _ptr(m, _u8p), M, _ptr(y), ctypes.byref(imag), threads)
    if rc:
        raise ValueError(f"oracle_fft_conv failed ({rc})")
    return (y, imag.value) if return_imag else y


def masked_filter(k_row, N: int, mask_row, lib=None):
    """k' = Re IFFT(mask * FFT(pad(k, 2N))), length 2N."""
    lib = lib or load()
    k_row = _f64(k_row)
    m = np.ascontiguousarray(mask_row, dtype=np.uint8)
    kp = np.empty(2 * N, dtype=np.float64)
    rc = lib.oracle_masked_filter(_ptr(k_row), k_row.size, N, _ptr(m, _u8p), _ptr(kp))
    if rc:
        raise ValueError("oracle_masked_filter: bad arguments")
    return kp


def circular_points(u_row, kp, ts, w_row=None, v_row=None, lib=None):
    """Masked output of one sequence at times ts through the circular form."""
    lib = lib or load()
    u_row, w_row, v_row, kp = _f64(u_row), _f64(w_row), _f64(v_row), _f64(kp)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    out = np.empty(ts.size, dtype=np.float64)
    rc = lib.oracle_circular_points(_ptr(u_row), _ptr(w_row), _ptr(v_row), _ptr(kp),
                                    u_row.size, _ptr(ts, _i64p), ts.size, _ptr(out))
    if rc:
        raise ValueError("oracle_circular_points: bad arguments")
    return out


# ---------------------------------------------------------------- backward
# Gradients of the scalar sum(dy * y) for y = v * conv(u * w, k) (FlashFFTConv
# summary page: the convolutions are trained, so the operator's backward pass
# is part of what a user runs; "Approach" gives the frequency-sparse filter).
# With x = u * w and g = v * dy:
#   dv[t] = dy[t] c[t],        c = conv(x, k) (no output gate)
#   dx[n] = sum_t g[t] k[t - n]            (correlation: the adjoint of conv)
#   du = dx * w,  dw = dx * u
#   dk[s] = sum_b sum_t g[t] x[t - s],     s < L
# With a frequency mask the filter acts as the 2N-periodic kp = Re IFFT(m FFT
# pad(k)) (see fft_conv); that operator is a real symmetric circulant, so
# dk = [Re IFFT(m FFT(r))][:L] with r the 2N-point circular correlation of g
# and x summed over the batch.  Gates that are absent (None) have no gradient.

def direct_bwd(u, k, dy, w=None, v=None):
    """Route D gradients (du, dk, dw, dv) by the sums above; no mask.

    u, w, v, dy: (B, H, N); k: (H, L).  Returns float64 arrays; dw / dv are
    None when w / v are absent."""
    u, k, dy = _f64(u), _f64(k), _f64(dy)
    w, v = _f64(w), _f64(v)
    B, H, N = u.shape
    L = k.shape[1]
    x = u * w if w is not None else u.copy()
    g = dy * v if v is not None else dy.copy()
    dv = None
    if v is not None:
        c = direct(u, k, w, None)
        dv = dy * c
    dx = np.zeros((B, H, N))
    dk = np.zeros((H, L))
    for s in range(L):
        # dx[n] += k[s] g[n + s] for n + s < N;  dk[s] = sum_b sum_t g[t] x[t - s]
        dx[:, :, :N - s] += k[None, :, s, None] * g[:, :, s:]
        dk[:, s] = np.sum(g[:, :, s:] * x[:, :, :N - s], axis=(0, 2))
    du = dx * w if w is not None else dx
    dw = dx * u if w is not None else None
    return du, dk, dw, dv


def _bin_keep(mask_row, N: int) -> np.ndarray:
    """Kept flag of each bin f < 2N: bin f follows its mirror 2N - f; rfft bins
    [0, N] form 128 blocks of N/128 bins and the Nyquist bin joins block 127."""
    M = 2 * N
    f = np.arange(M)
    fr = np.where(f <= N, f, M - f)
    blk = np.minimum(fr // (N // 128), 127)
    return np.asarray(mask_row, dtype=np.uint8)[blk] != 0


def fft_bwd(u, k, dy, w=None, v=None, mask=None, lib=None):
    """Route F gradients through the oracle's FFT (2N points), optional (H, 128) mask."""
    u, k, dy = _f64(u), _f64(k), _f64(dy)
    w, v = _f64(w), _f64(v)
    B, H, N = u.shape
    L = k.shape[1]
    M = 2 * N
    x = u * w if w is not None else u.copy()
    g = dy * v if v is not None else dy.copy()
    dx = np.empty((B, H, N))
    c = np.empty((B, H, N))
    dk = np.empty((H, L))
    for h in range(H):
        kpad = np.zeros(M)
        kpad[:L] = k[h]
        K = fft(kpad, -1, lib)
        keep = np.ones(M, dtype=bool) if mask is None else _bin_keep(mask[h], N)
        K = np.where(keep, K, 0.0)
        R = np.zeros(M, dtype=np.complex128)
        for b in range(B):
            xp = np.zeros(M)
            xp[:N] = x[b, h]
            gp = np.zeros(M)
            gp[:N] = g[b, h]
            X = fft(xp, -1, lib)
            G = fft(gp, -1, lib)
            c[b, h] = fft(X * K, +1, lib).real[:N] / M
            dx[b, h] = fft(G * np.conj(K), +1, lib).real[:N] / M
            R += G * np.conj(X)
        dk[h] = fft(np.where(keep, R, 0.0), +1, lib).real[:L] / M
    du = dx * w if w is not None else dx
    dw = dx * u if w is not None else None
    dv = dy * c if v is not None else None
    return du, dk, dw, dv


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 in float64 (b is the oracle's value); ||a - b||_2
    when b is all zero."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.sqrt(np.sum(b * b))
    num = np.sqrt(np.sum((a - b) ** 2))
    return float(num / den) if den > 0 else float(num)


def seq_rel_l2(a, b) -> np.ndarray:
    """rel_l2 of every sequence: the last axis is the sequence, the leading axes
    (for a (B, H, N) tensor: b and h) are flattened.  One value per sequence, in
    row-major order of the leading axes; a 1-D input is one sequence."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}")
    n = a.shape[-1] if a.ndim else 1
    a2 = a.reshape(-1, n)
    b2 = b.reshape(-1, n)
    den = np.sqrt(np.sum(b2 * b2, axis=1))
    num = np.sqrt(np.sum((a2 - b2) ** 2, axis=1))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def max_abs(a, b) -> float:
    """max |a - b| over all elements (0 for empty inputs)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}")
    return float(np.max(np.abs(a - b))) if a.size else 0.0
