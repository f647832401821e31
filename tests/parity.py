"""Comparison of a GPU result with the oracle's, shared by every GPU parity test.

The method computes exact convolutions per (batch row, channel) sequence
(FlashFFTConv summary page, "Summary"), so a result is accepted only when
  - every element is finite,
  - the relative L2 error over the whole compared tensor is within tol, and
  - the worst relative L2 error of any single sequence (the last axis; the
    leading axes are flattened) is within seq_tol (default: tol),
and the max-abs error is printed, absolute and as a fraction of max|ref|.
The per-sequence bound is what catches one wrong sequence among many: over
49,152 sequences a sequence of zeros moves the whole-tensor error by only
1/sqrt(49152) = 4.5e-3.
"""
from __future__ import annotations

import os

import numpy as np

import oracle


def _label(what: str) -> str:
    if what:
        return what
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0] or "result"


def metrics(got, ref) -> dict:
    """relL2 over everything, per-sequence relL2 (worst and its index), max-abs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != oracle shape {ref.shape}")
    seqs = oracle.seq_rel_l2(got, ref) if got.size else np.zeros(0)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    mabs = oracle.max_abs(got, ref)
    return {
        "rel_l2": oracle.rel_l2(got, ref) if got.size else 0.0,
        "worst_seq_rel_l2": float(np.max(seqs)) if seqs.size else 0.0,
        "worst_seq": int(np.argmax(seqs)) if seqs.size else -1,
        "n_seq": int(seqs.size),
        "max_abs": mabs,
        "max_abs_rel": mabs / scale if scale > 0 else mabs,
        "finite": bool(np.all(np.isfinite(got))),
    }


def check(got, ref, tol: float, what: str = "", seq_tol: float | None = None) -> dict:
    """Assert the three conditions of the module docstring; returns the metrics."""
    m = metrics(got, ref)
    name = _label(what)
    print(f"[parity] {name}: relL2 {m['rel_l2']:.3e}, worst sequence relL2 {m['worst_seq_rel_l2']:.3e} "
          f"(sequence {m['worst_seq']} of {m['n_seq']}), max-abs {m['max_abs']:.3e} "
          f"({m['max_abs_rel']:.3e} of max|ref|)", flush=True)
    assert m["finite"], f"{name}: non-finite values in the result"
    assert m["rel_l2"] <= tol, f"{name}: relL2 {m['rel_l2']:.3e} > {tol:.1e}"
    bound = tol if seq_tol is None else seq_tol
    assert m["worst_seq_rel_l2"] <= bound, (
        f"{name}: sequence {m['worst_seq']} has relL2 {m['worst_seq_rel_l2']:.3e} > {bound:.1e}")
    return m
