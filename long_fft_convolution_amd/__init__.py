"""MI355X (gfx950) exact long causal FFT convolution -- Python binding.

Thin ctypes layer over the C ABI of ``libfftconv.so`` (include/fftconv.h):
every function has the C function's name and only marshals arguments.
torch tensors supply device memory and the current HIP stream; every step of
the convolution runs in the library's HIP kernels.  There is no CPU fallback:
if the library is not built, importing the functions raises.

    y[b,h,t] = v[b,h,t] * sum_{s<=min(t,L-1)} k[h,s] * u[b,h,t-s] * w[b,h,t-s]

(FlashFFTConv summary page: exact FFT convolution, gated, with partial and
frequency-sparse filters.)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loads torch's HIP runtime first, so the library shares it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfftconv.so")

FFTCONV_F32, FFTCONV_F16, FFTCONV_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FFTCONV_F32, torch.float16: FFTCONV_F16, torch.bfloat16: FFTCONV_BF16}
STATUS = {0: "FFTCONV_OK", 1: "FFTCONV_ERR_INVALID_ARGUMENT", 2: "FFTCONV_ERR_UNSUPPORTED",
          3: "FFTCONV_ERR_WORKSPACE", 4: "FFTCONV_ERR_FILTER_MISMATCH", 5: "FFTCONV_ERR_HIP"}

_lib = None


class FFTConvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_fft_convolution_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.fftconv_filter_bytes.argtypes = [i64, i64, ctypes.c_int]
    lib.fftconv_filter_bytes.restype = sz
    lib.fftconv_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fftconv_workspace_bytes.restype = sz
    lib.fftconv_mask_blocks.argtypes = [i64]
    lib.fftconv_mask_blocks.restype = i64
    lib.fftconv_prepare_filter.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp, sz, vp, sz, vp]
    lib.fftconv_prepare_filter.restype = ctypes.c_int
    lib.fftconv_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, vp, sz, vp]
    lib.fftconv_fwd.restype = ctypes.c_int
    lib.fftconv_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, vp]
    lib.fftconv_fwd_noalloc.restype = ctypes.c_int
    lib.fftconv_fwd_noalloc_scratch_bytes.argtypes = []
    lib.fftconv_fwd_noalloc_scratch_bytes.restype = sz
    lib.fftconv_fwd_taps_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fftconv_fwd_taps_workspace_bytes.restype = sz
    lib.fftconv_fwd_taps.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, vp, sz, vp]
    lib.fftconv_fwd_taps.restype = ctypes.c_int
    lib.fftconv_bwd_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fftconv_bwd_workspace_bytes.restype = sz
    lib.fftconv_bwd.argtypes = [vp] * 9 + [i64, i64, i64, i64, vp, ctypes.c_int, vp, sz, vp]
    lib.fftconv_bwd.restype = ctypes.c_int
    lib.fftconv_init.argtypes = []
    lib.fftconv_init.restype = ctypes.c_int
    lib.fftconv_status_string.argtypes = [ctypes.c_int]
    lib.fftconv_status_string.restype = ctypes.c_char_p
    lib.fftconv_last_error.argtypes = []
    lib.fftconv_last_error.restype = ctypes.c_char_p
    lib.fftconv_export_filter_rfft.argtypes = [vp, i64, i64, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_double), vp]
    lib.fftconv_export_filter_rfft.restype = ctypes.c_int
    lib.fftconv_short_filter_bytes.argtypes = [i64, ctypes.c_int]
    lib.fftconv_short_filter_bytes.restype = sz
    lib.fftconv_prepare_short_filter.argtypes = [vp, i64, i64, ctypes.c_int, vp, sz, vp]
    lib.fftconv_prepare_short_filter.restype = ctypes.c_int
    lib.fftconv_fwd_short.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.fftconv_fwd_short.restype = ctypes.c_int
    lib.fftconv_bwd_short.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_int, vp]
    lib.fftconv_bwd_short.restype = ctypes.c_int
    lib.fftconv_eqlinear_weight_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fftconv_eqlinear_weight_bytes.restype = sz
    lib.fftconv_eqlinear_prepare.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp, sz, vp]
    lib.fftconv_eqlinear_prepare.restype = ctypes.c_int
    lib.fftconv_eqlinear_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.fftconv_eqlinear_fwd.restype = ctypes.c_int
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises ImportError when not built)."""
    return _load()


def _check(status: int):
    if status != 0:
        raise FFTConvError(status, _load().fftconv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_tensor(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dtype_code(dtype: torch.dtype) -> int:
    return _DTYPE_CODE[dtype]


def fftconv_filter_bytes(H: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_filter_bytes(H, N, code))


def fftconv_workspace_bytes(B: int, H: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_workspace_bytes(B, H, N, code))


def fftconv_mask_blocks(N: int) -> int:
    return int(_load().fftconv_mask_blocks(N))


def fftconv_init(device=None) -> None:
    """Build the library's constant tables on `device` (default: the current one); synchronous."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(_load().fftconv_init())


def fftconv_status_string(status: int) -> str:
    return _load().fftconv_status_string(status).decode()


def fftconv_last_error() -> str:
    return _load().fftconv_last_error().decode()


def fftconv_prepare_filter(k: torch.Tensor, N: int, K_f: torch.Tensor,
                           workspace: torch.Tensor | None = None, stream=None) -> None:
    """K_f <- prepared spectrum of the (H, L) filter k for sequence length N."""
    _dev_tensor(k, "k")
    _dev_tensor(K_f, "K_f")
    _dev_tensor(workspace, "workspace")
    H, L = k.shape
    _check(_load().fftconv_prepare_filter(
        _ptr(k), H, L, N, dtype_code(k.dtype), _ptr(K_f), K_f.numel() * K_f.element_size(),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream, k.device)))


def fftconv_fwd(u: torch.Tensor, K_f: torch.Tensor, w: torch.Tensor | None,
                v: torch.Tensor | None, out: torch.Tensor, L_filter: int,
                sparsity_mask: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> None:
    """out <- v * causal_conv(u * w, k) through the prepared filter K_f."""
    for name, t in (("u", u), ("K_f", K_f), ("w", w), ("v", v), ("out", out),
                    ("sparsity_mask", sparsity_mask), ("workspace", workspace)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_fwd(
        _ptr(u), _ptr(K_f), _ptr(w), _ptr(v), _ptr(out), B, H, N, L_filter, _ptr(sparsity_mask),
        dtype_code(u.dtype), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream, u.device)))


def fftconv_fwd_noalloc(u: torch.Tensor, K_f: torch.Tensor, w: torch.Tensor | None,
                        v: torch.Tensor | None, out: torch.Tensor, L_filter: int,
                        sparsity_mask: torch.Tensor | None = None, stream=None) -> None:
    """fftconv_fwd with the library's static scratch instead of a workspace (after fftconv_init)."""
    for name, t in (("u", u), ("K_f", K_f), ("w", w), ("v", v), ("out", out),
                    ("sparsity_mask", sparsity_mask)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_fwd_noalloc(
        _ptr(u), _ptr(K_f), _ptr(w), _ptr(v), _ptr(out), B, H, N, L_filter, _ptr(sparsity_mask),
        dtype_code(u.dtype), _stream(stream, u.device)))


def fftconv_fwd_noalloc_scratch_bytes() -> int:
    return int(_load().fftconv_fwd_noalloc_scratch_bytes())


def fftconv_fwd_taps_workspace_bytes(B: int, H: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_fwd_taps_workspace_bytes(B, H, N, code))


def fftconv_fwd_taps(u: torch.Tensor, k: torch.Tensor, w: torch.Tensor | None,
                     v: torch.Tensor | None, out: torch.Tensor, workspace: torch.Tensor,
                     sparsity_mask: torch.Tensor | None = None, stream=None) -> None:
    """out <- v * causal_conv(u * w, k) from the (H, L) taps k, transformed within the call."""
    for name, t in (("u", u), ("k", k), ("w", w), ("v", v), ("out", out),
                    ("sparsity_mask", sparsity_mask), ("workspace", workspace)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_fwd_taps(
        _ptr(u), _ptr(k), _ptr(w), _ptr(v), _ptr(out), B, H, N, k.shape[1], _ptr(sparsity_mask),
        dtype_code(u.dtype), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream, u.device)))


def fftconv_bwd_workspace_bytes(B: int, H: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_bwd_workspace_bytes(B, H, N, code))


def fftconv_bwd(dy: torch.Tensor, u: torch.Tensor, K_f: torch.Tensor, w: torch.Tensor | None,
                v: torch.Tensor | None, du: torch.Tensor | None, dk: torch.Tensor | None,
                dw: torch.Tensor | None, dv: torch.Tensor | None, L_filter: int,
                sparsity_mask: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None) -> None:
    """Gradients of sum(dy * fftconv_fwd(u, K_f, w, v)) into du, dk, dw, dv (None = skip)."""
    for name, t in (("dy", dy), ("u", u), ("K_f", K_f), ("w", w), ("v", v), ("du", du), ("dk", dk),
                    ("dw", dw), ("dv", dv), ("sparsity_mask", sparsity_mask), ("workspace", workspace)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_bwd(
        _ptr(dy), _ptr(u), _ptr(K_f), _ptr(w), _ptr(v), _ptr(du), _ptr(dk), _ptr(dw), _ptr(dv),
        B, H, N, L_filter, _ptr(sparsity_mask), dtype_code(u.dtype), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream, u.device)))


def fftconv_export_filter_rfft(K_f: torch.Tensor, H: int, N: int, dtype, stream=None) -> np.ndarray:
    """Synchronous: natural-order rfft bins (H, N+1) complex128 decoded from K_f."""
    _dev_tensor(K_f, "K_f")
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    outbuf = np.empty((H, N + 1, 2), dtype=np.float64)
    _check(_load().fftconv_export_filter_rfft(
        _ptr(K_f), H, N, code, outbuf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        _stream(stream, K_f.device)))
    return outbuf[..., 0] + 1j * outbuf[..., 1]


# ---------------------------------------------------------------- plumbing
def fftconv_short_filter_bytes(H: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_short_filter_bytes(H, code))


def fftconv_prepare_short_filter(k: torch.Tensor, K_s: torch.Tensor, stream=None) -> None:
    """K_s <- spectrum of the (H, L) filter k, L <= 1024, for the chunked short-filter path."""
    _dev_tensor(k, "k")
    _dev_tensor(K_s, "K_s")
    H, L = k.shape
    _check(_load().fftconv_prepare_short_filter(
        _ptr(k), H, L, dtype_code(k.dtype), _ptr(K_s), K_s.numel() * K_s.element_size(),
        _stream(stream, k.device)))


def fftconv_fwd_short(u: torch.Tensor, K_s: torch.Tensor, w: torch.Tensor | None, v: torch.Tensor | None,
                      out: torch.Tensor, L_filter: int, stream=None) -> None:
    """out <- v * causal_conv(u * w, k) through the short-filter spectrum K_s (N a multiple of 1024)."""
    for name, t in (("u", u), ("K_s", K_s), ("w", w), ("v", v), ("out", out)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_fwd_short(
        _ptr(u), _ptr(K_s), _ptr(w), _ptr(v), _ptr(out), B, H, N, L_filter, dtype_code(u.dtype),
        _stream(stream, u.device)))


def fftconv_bwd_short(dy: torch.Tensor, u: torch.Tensor, K_s: torch.Tensor, w: torch.Tensor | None,
                      v: torch.Tensor | None, du: torch.Tensor | None, dk: torch.Tensor | None,
                      dw: torch.Tensor | None, dv: torch.Tensor | None, L_filter: int, stream=None) -> None:
    """Gradients of sum(dy * fftconv_fwd_short(u, K_s, w, v)) into du, dk, dw, dv (None = skip)."""
    for name, t in (("dy", dy), ("u", u), ("K_s", K_s), ("w", w), ("v", v), ("du", du), ("dk", dk),
                    ("dw", dw), ("dv", dv)):
        _dev_tensor(t, name)
    B, H, N = u.shape
    _check(_load().fftconv_bwd_short(
        _ptr(dy), _ptr(u), _ptr(K_s), _ptr(w), _ptr(v), _ptr(du), _ptr(dk), _ptr(dw), _ptr(dv),
        B, H, N, L_filter, dtype_code(u.dtype), _stream(stream, u.device)))


def causal_conv_short(u, k, w=None, v=None, stream=None):
    """Prepare a short filter k (L <= 1024) and run one chunked forward call."""
    H, L = k.shape
    K_s = torch.empty(fftconv_short_filter_bytes(H, u.dtype), dtype=torch.uint8, device=u.device)
    fftconv_prepare_short_filter(k, K_s, stream)
    out = torch.empty_like(u)
    fftconv_fwd_short(u, K_s, w, v, out, L, stream)
    return out


def causal_conv_short_bwd(u, k, dy, w=None, v=None, stream=None):
    """Prepare a short filter k and run one backward call; returns (du, dk, dw, dv)."""
    H, L = k.shape
    K_s = torch.empty(fftconv_short_filter_bytes(H, u.dtype), dtype=torch.uint8, device=u.device)
    fftconv_prepare_short_filter(k, K_s, stream)
    du = torch.empty_like(u)
    dk = torch.empty((H, L), dtype=u.dtype, device=u.device)
    dw = torch.empty_like(u) if w is not None else None
    dv = torch.empty_like(u) if v is not None else None
    fftconv_bwd_short(dy, u, K_s, w, v, du, dk, dw, dv, L, stream)
    return du, dk, dw, dv


def fftconv_eqlinear_weight_bytes(T: int, C_out: int, C_in: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(_load().fftconv_eqlinear_weight_bytes(T, C_out, C_in, code))


def fftconv_eqlinear_prepare(W: torch.Tensor, W_f: torch.Tensor, stream=None) -> None:
    """W_f <- the group-axis real DFT of W (T, C_out, C_in)."""
    _dev_tensor(W, "W")
    _dev_tensor(W_f, "W_f")
    T, C_out, C_in = W.shape
    _check(_load().fftconv_eqlinear_prepare(
        _ptr(W), T, C_out, C_in, dtype_code(W.dtype), _ptr(W_f), W_f.numel() * W_f.element_size(),
        _stream(stream, W.device)))


def fftconv_eqlinear_fwd(x: torch.Tensor, W_f: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """y (N, T, C_out) <- group circular convolution of x (N, T, C_in) with the prepared W_f."""
    for name, t in (("x", x), ("W_f", W_f), ("y", y)):
        _dev_tensor(t, name)
    N, T, C_in = x.shape
    C_out = y.shape[2]
    _check(_load().fftconv_eqlinear_fwd(
        _ptr(x), _ptr(W_f), _ptr(y), N, T, C_in, C_out, dtype_code(x.dtype), _stream(stream, x.device)))


def eqlinear(x, W, stream=None):
    """Prepare W and run the group convolution once (allocations by torch)."""
    T, C_out, C_in = W.shape
    W_f = torch.empty(fftconv_eqlinear_weight_bytes(T, C_out, C_in, W.dtype), dtype=torch.uint8, device=x.device)
    fftconv_eqlinear_prepare(W, W_f, stream)
    y = torch.empty((x.shape[0], T, C_out), dtype=x.dtype, device=x.device)
    fftconv_eqlinear_fwd(x, W_f, y, stream)
    return y


def alloc_filter(H: int, N: int, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Device buffer for K_f (torch allocation; the library never allocates it)."""
    return torch.empty(fftconv_filter_bytes(H, N, dtype), dtype=torch.uint8, device=device)


def alloc_workspace(B: int, H: int, N: int, dtype: torch.dtype, device="cuda"):
    n = fftconv_workspace_bytes(B, H, N, dtype)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def causal_conv(u, k, w=None, v=None, sparsity_mask=None, stream=None):
    """Prepare k and run one forward call (allocations by torch)."""
    B, H, N = u.shape
    L = k.shape[1]
    K_f = alloc_filter(H, N, u.dtype, u.device)
    ws_p = alloc_workspace(1, H, N, u.dtype, u.device)
    fftconv_prepare_filter(k, N, K_f, ws_p, stream)
    ws = alloc_workspace(B, H, N, u.dtype, u.device)
    out = torch.empty_like(u)
    fftconv_fwd(u, K_f, w, v, out, L, sparsity_mask, ws, stream)
    return out


def causal_conv_bwd(u, k, dy, w=None, v=None, sparsity_mask=None, stream=None):
    """Prepare k and run one backward call; returns (du, dk, dw, dv), None for absent gates."""
    B, H, N = u.shape
    L = k.shape[1]
    K_f = alloc_filter(H, N, u.dtype, u.device)
    ws_p = alloc_workspace(1, H, N, u.dtype, u.device)
    fftconv_prepare_filter(k, N, K_f, ws_p, stream)
    ws = torch.empty(fftconv_bwd_workspace_bytes(B, H, N, u.dtype), dtype=torch.uint8, device=u.device)
    du = torch.empty_like(u)
    dk = torch.empty((H, L), dtype=u.dtype, device=u.device)
    dw = torch.empty_like(u) if w is not None else None
    dv = torch.empty_like(u) if v is not None else None
    fftconv_bwd(dy, u, K_f, w, v, du, dk, dw, dv, L, sparsity_mask, ws, stream)
    return du, dk, dw, dv
