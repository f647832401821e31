"""Seeded synthetic inputs for the causal long-convolution workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the convolution's arithmetic, so both the HIP path and the
CPU oracle may use it.

Workloads (the FlashFFTConv summary page's measured settings, with the
shapes, precisions and distributions fixed here because the page gives none):

=====================  ====  ======  =========  =========  =====  ======  =====
name                   B     H       N          L          dtype  gated   mask
=====================  ====  ======  =========  =========  =====  ======  =====
ungated_fp32_n1k       1     4       1,024      1,024      f32    no      --
gated_fp16_n1k         64    768     1,024      1,024      f16    yes     --
gated_bf16_n16k        4     2,560   16,384     16,384     bf16   yes     --
ungated_fp16_n1m       1     256     1,048,576  1,048,576  f16    no      --
partial_sparse_n4m     1     128     4,194,304  1,048,576  f16    no      79 %
=====================  ====  ======  =========  =========  =====  ======  =====

Distributions: u, w, v ~ N(0, 1).  Filter k[h, t] = N(0, 1) * exp(-alpha_h t)
with alpha_h = 10**U(-4, -1) (log-uniform in [1e-4, 1e-1]), except the small
fp32 workload, whose filter is N(0, 1) * exp(-0.01 t).  The frequency mask of
the partial workload zeroes blocks 27..127 of 128 (the high-frequency 78.9 %
of the rfft bins) for every channel.

Draw order, from numpy ``default_rng(seed)``: filter noise (H, L), alpha (H),
u, w, v; each in float64, then rounded to the storage dtype by torch
(round-to-nearest-even).  Large tensors are drawn channel-block by
channel-block from the same generator so memory stays bounded; the stream of
numbers is the same as one big draw in C order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    L: int
    dtype: str
    gated: bool
    decay: str = "loguniform"     # or "fixed0.01"
    mask_keep_blocks: int | None = None  # blocks [0, keep) kept, the rest zeroed
    seed: int = 1000
    short: bool = False                  # run through the chunked short-filter path (L <= 1024)

    @property
    def elems(self) -> int:
        return self.B * self.H * self.N


WORKLOADS = {
    w.name: w for w in [
        Workload("ungated_fp32_n1k", 1, 4, 1024, 1024, "f32", False, "fixed0.01", None, 1000),
        Workload("gated_fp16_n1k", 64, 768, 1024, 1024, "f16", True, "loguniform", None, 1001),
        Workload("gated_bf16_n16k", 4, 2560, 16384, 16384, "bf16", True, "loguniform", None, 1002),
        Workload("ungated_fp16_n1m", 1, 256, 1 << 20, 1 << 20, "f16", False, "loguniform", None, 1003),
        Workload("partial_sparse_n4m", 1, 128, 1 << 22, 1 << 20, "f16", False, "loguniform", 27, 1004),
        # the chunked short-filter path: a 512-tap filter on the 1M-point sequences
        Workload("short_fp16_n1m_l512", 1, 256, 1 << 20, 512, "f16", False, "loguniform", None, 1005, True),
    ]
}


@dataclass
class Inputs:
    """Storage-dtype tensors on the host (CPU); w, v are None when ungated."""
    u: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor | None
    v: torch.Tensor | None
    mask: np.ndarray | None           # (H, 128) uint8 or None
    meta: dict = field(default_factory=dict)

    def f64(self, name: str):
        t = getattr(self, name)
        return None if t is None else t.to(torch.float64).numpy()


def _normal_rounded(rng, shape, dtype, chunk_rows: int = 8):
    """Draw N(0,1) float64 of `shape` in C order, rounding each chunk to dtype."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1, shape[-1])
    rows = flat.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        flat[r0:r1] = torch.from_numpy(rng.standard_normal((r1 - r0, shape[-1])))
    return out


def make_filter(rng, H: int, L: int, decay: str) -> np.ndarray:
    """k[h, t] = N(0,1) * exp(-alpha_h * t) in float64 (noise drawn before alpha)."""
    noise = rng.standard_normal((H, L))
    if decay == "fixed0.01":
        alpha = np.full(H, 0.01)
    else:
        alpha = 10.0 ** rng.uniform(-4.0, -1.0, size=H)
    t = np.arange(L, dtype=np.float64)
    for h in range(H):
        noise[h] *= np.exp(-alpha[h] * t)
    return noise


def band_mask(H: int, keep_blocks: int, nblocks: int = 128) -> np.ndarray:
    """Contiguous low-frequency band kept: blocks [0, keep) = 1, the rest 0."""
    m = np.zeros((H, nblocks), dtype=np.uint8)
    m[:, :keep_blocks] = 1
    return m


def random_mask(H: int, seed: int, keep_prob: float = 0.5, nblocks: int = 128) -> np.ndarray:
    """Seeded random block mask (test variant)."""
    rng = np.random.default_rng(seed)
    return (rng.random((H, nblocks)) < keep_prob).astype(np.uint8)


def generate(B: int, H: int, N: int, L: int, dtype: str = "f32", gated: bool = False,
             decay: str = "loguniform", seed: int = 0,
             mask_keep_blocks: int | None = None) -> Inputs:
    """Seeded inputs rounded to the storage dtype (host tensors)."""
    tdt = DTYPES[dtype]
    rng = np.random.default_rng(seed)
    k64 = make_filter(rng, H, L, decay)
    k = torch.from_numpy(k64).to(tdt)
    del k64
    u = _normal_rounded(rng, (B, H, N), tdt)
    w = v = None
    if gated:
        w = _normal_rounded(rng, (B, H, N), tdt)
        v = _normal_rounded(rng, (B, H, N), tdt)
    mask = None if mask_keep_blocks is None else band_mask(H, mask_keep_blocks)
    return Inputs(u=u, k=k, w=w, v=v, mask=mask,
                  meta=dict(B=B, H=H, N=N, L=L, dtype=dtype, gated=gated, decay=decay,
                            seed=seed, mask_keep_blocks=mask_keep_blocks))


def generate_workload(name: str, seed: int | None = None) -> Inputs:
    w = WORKLOADS[name]
    return generate(w.B, w.H, w.N, w.L, w.dtype, w.gated, w.decay,
                    w.seed if seed is None else seed, w.mask_keep_blocks)


# ---- group-axis circular convolution (the Flash EQ-Linear operator) ----------
@dataclass(frozen=True)
class EqWorkload:
    name: str
    N: int        # tokens
    T: int        # cyclic group order
    C_in: int
    C_out: int
    dtype: str
    seed: int


EQ_WORKLOADS = {
    w.name: w for w in [
        # a vision-transformer-sized equivariant linear layer: 64K tokens, C8 rotations, 128 channels
        EqWorkload("eqlinear_fp16_t8", 65536, 8, 128, 128, "f16", 1006),
        # the same layer in fp32 storage and arithmetic
        EqWorkload("eqlinear_fp32_t8", 65536, 8, 128, 128, "f32", 1007),
    ]
}


def generate_eq(name: str):
    """x (N, T, C_in) ~ N(0, 1) and W (T, C_out, C_in) ~ N(0, 1 / (T C_in)), rounded to the dtype."""
    w = EQ_WORKLOADS[name]
    g = torch.Generator().manual_seed(w.seed)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    x = torch.randn((w.N, w.T, w.C_in), generator=g).to(dt)
    W = (torch.randn((w.T, w.C_out, w.C_in), generator=g) / float(np.sqrt(w.T * w.C_in))).to(dt)
    return x, W
