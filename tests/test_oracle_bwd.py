"""Pins of the oracle's backward pass (CPU).

The gradients are pinned to the definition of a gradient, through the forward
routes that test_oracle.py pins independently: L(theta) = sum(dy * y(theta)) is
linear in each of u, w, v and k on its own, so the central difference
(L(theta + e_i) - L(theta - e_i)) / 2 equals dL/dtheta_i up to rounding, for
every entry i.  The masked case goes through the masked forward route.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, H, N, L, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N)), rng.standard_normal((H, L)), rng.standard_normal((B, H, N)),
            rng.standard_normal((B, H, N)), rng.standard_normal((B, H, N)))


def _loss(fwd, u, k, w, v, dy):
    return float(np.sum(dy * fwd(u, k, w, v)))


def _fd_grad(fwd, args, name, dy):
    """Central differences with step 1 over every entry of args[name]."""
    a = dict(args)
    base = a[name]
    grad = np.empty_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        p, m = base.copy(), base.copy()
        p[i] += 1.0
        m[i] -= 1.0
        a[name] = p
        lp = _loss(fwd, a["u"], a["k"], a["w"], a["v"], dy)
        a[name] = m
        lm = _loss(fwd, a["u"], a["k"], a["w"], a["v"], dy)
        grad[i] = 0.5 * (lp - lm)
    return grad


@pytest.mark.parametrize("gates", ["both", "none", "w", "v"])
def test_direct_bwd_matches_finite_differences(gates):
    B, H, N, L = 2, 2, 12, 5
    u, k, w, v, dy = _inputs(B, H, N, L, seed=11)
    w = w if gates in ("both", "w") else None
    v = v if gates in ("both", "v") else None
    du, dk, dw, dv = oracle.direct_bwd(u, k, dy, w, v)
    fwd = lambda u_, k_, w_, v_: oracle.direct(u_, k_, w_, v_)
    args = {"u": u, "k": k, "w": w, "v": v}
    pairs = [("u", du), ("k", dk)] + ([("w", dw)] if w is not None else []) + ([("v", dv)] if v is not None else [])
    for name, got in pairs:
        want = _fd_grad(fwd, args, name, dy)
        assert np.max(np.abs(got - want)) < 1e-10 * max(1.0, np.max(np.abs(want))), name
    if w is None:
        assert dw is None
    if v is None:
        assert dv is None


@pytest.mark.parametrize("kind", ["none", "band", "random"])
def test_fft_bwd_matches_finite_differences_masked(kind):
    # N = 128 is the smallest size with one bin per mask block
    B, H, N, L = 1, 2, 128, 40
    u, k, w, v, dy = _inputs(B, H, N, L, seed=12)
    rng = np.random.default_rng(5)
    mask = None
    if kind == "band":
        mask = np.zeros((H, 128), np.uint8)
        mask[:, :27] = 1
    elif kind == "random":
        mask = (rng.random((H, 128)) < 0.6).astype(np.uint8)
    du, dk, dw, dv = oracle.fft_bwd(u, k, dy, w, v, mask)
    fwd = lambda u_, k_, w_, v_: oracle.fft_conv(u_, k_, w_, v_, mask=mask)
    args = {"u": u, "k": k, "w": w, "v": v}
    # every entry of k, and a seeded sample of the entries of u, w, v (the full
    # set would take 2 * 128 forward transforms per array)
    want_k = _fd_grad(fwd, args, "k", dy)
    assert np.max(np.abs(dk - want_k)) < 1e-9 * np.max(np.abs(want_k))
    for name, got in (("u", du), ("w", dw), ("v", dv)):
        base = args[name]
        for t in rng.integers(0, N, 6):
            h = int(rng.integers(0, H))
            p, m = base.copy(), base.copy()
            p[0, h, t] += 1.0
            m[0, h, t] -= 1.0
            a = dict(args)
            a[name] = p
            lp = _loss(fwd, a["u"], a["k"], a["w"], a["v"], dy)
            a[name] = m
            lm = _loss(fwd, a["u"], a["k"], a["w"], a["v"], dy)
            want = 0.5 * (lp - lm)
            assert abs(got[0, h, t] - want) < 1e-9 * max(1.0, abs(want)), (name, h, t)


def test_routes_agree_unmasked():
    B, H, N, L = 2, 3, 256, 100
    u, k, w, v, dy = _inputs(B, H, N, L, seed=13)
    a = oracle.direct_bwd(u, k, dy, w, v)
    b = oracle.fft_bwd(u, k, dy, w, v)
    for x, y in zip(a, b):
        assert oracle.rel_l2(y, x) < 1e-12


def test_delta_filter_gradients_are_gates():
    # k = delta: y = v u w, so du = dy v w, dw = dy v u, dv = dy u w, dk[0] = sum dy v u w
    B, H, N = 2, 2, 64
    u, _, w, v, dy = _inputs(B, H, N, 1, seed=14)
    k = np.ones((H, 1))
    du, dk, dw, dv = oracle.direct_bwd(u, k, dy, w, v)
    assert np.allclose(du, dy * v * w, atol=1e-13)
    assert np.allclose(dw, dy * v * u, atol=1e-13)
    assert np.allclose(dv, dy * u * w, atol=1e-13)
    assert np.allclose(dk[:, 0], np.sum(dy * v * u * w, axis=(0, 2)), atol=1e-11)
