"""Planted-mistake checks for the oracle's pins (CPU only).

Each case copies the oracle's C source, plants one plausible mistake (a
dropped term, a flipped sign, a wrong index or stride, a swapped operand),
compiles the copy into a temporary library and runs a compact set of the
pins from test_oracle.py against it.  The unmodified oracle must pass every
pin; every mutant must fail at least one.  Nothing here touches the GPU or
the HIP library.
"""
import os
import shutil

import numpy as np
import pytest

import oracle

MUTANTS = {
    "fft_twiddle_sign": ("double ang = (double)sign * ORACLE_PI", "double ang = (double)(-sign) * ORACLE_PI"),
    "fft_butterfly_sign": ("re[q] = re[s] - br;", "re[q] = re[s] + br;"),
    "direct_drops_last_tap": ("for (int64_t s = 0; s <= smax; ++s) {", "for (int64_t s = 0; s < smax; ++s) {"),
    "direct_gate_swapped": ("double x = u[t - s] * (w ? w[t - s] : 1.0);", "double x = u[t - s] * (v ? v[t - s] : 1.0);"),
    # filter read as the transposed (L, H) array: a wrong-layout mistake that
    # stays inside the buffer (a wrong stride that reads past it would make
    # the mutant's output undefined rather than wrong)
    "points_filter_stride": ("acc += k[h * L + s] * (us[t - s]", "acc += k[s * H + h] * (us[t - s]"),
    "fft_conv_correlation": ("xr[f] = a * kr[f] - bq * ki[f];", "xr[f] = a * kr[f] + bq * ki[f];"),
    "fft_conv_normalisation": ("(xr[t] / (double)M);", "(xr[t] / (double)N);"),
    "fft_conv_circular_input": ("xr[n] = n < N ? us[n] * (ws ? ws[n] : 1.0) : 0.0;",
                                "xr[n] = us[n % N] * (ws ? ws[n % N] : 1.0);"),
    "mask_mirror_index": ("int64_t fr = f <= N ? f : M - f; /* Hermitian", "int64_t fr = f <= N ? f : f - N; /* Hermitian"),
    "mask_block_off_by_one": ("int64_t b = f / G;", "int64_t b = (f + 1) / G;"),
    "masked_filter_no_mirror": ("        int64_t fr = f <= N ? f : M - f;\n        if (!bin_kept(mask_row",
                                "        int64_t fr = f <= N ? f : f;\n        if (fr > N) continue;\n        if (!bin_kept(mask_row"),
}


def _pins_hold(lib) -> list:
    """Compact pin set; returns the names of the pins that fail."""
    failed = []
    rng = np.random.default_rng(1)

    def rel(a, b):
        return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)

    # FFT vs brute-force DFT, both signs
    M = 64
    x = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    n = np.arange(M)
    for sign in (-1, 1):
        ref = np.array([np.sum(x * np.exp(sign * 2j * np.pi * f * n / M)) for f in range(M)])
        if rel(oracle.fft(x, sign, lib=lib), ref) > 1e-12:
            failed.append(f"fft_bruteforce{sign}")
    # direct and FFT routes vs numpy.convolve, gated, partial filter
    B, H, N, L = 2, 3, 256, 40
    u = rng.standard_normal((B, H, N))
    w = rng.standard_normal((B, H, N))
    v = rng.standard_normal((B, H, N))
    k = rng.standard_normal((H, L))
    ref = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            ref[b, h] = np.convolve(u[b, h] * w[b, h], k[h])[:N] * v[b, h]
    if rel(oracle.direct(u, k, w, v, lib=lib), ref) > 1e-13:
        failed.append("direct_vs_convolve")
    if rel(oracle.fft_conv(u, k, w, v, lib=lib), ref) > 1e-12:
        failed.append("fft_vs_convolve")
    pts = np.stack([rng.integers(0, B, 30), rng.integers(0, H, 30), rng.integers(0, N, 30)], 1)
    if rel(oracle.direct_points(u, k, pts, w, v, lib=lib), ref[pts[:, 0], pts[:, 1], pts[:, 2]]) > 1e-13:
        failed.append("points_vs_convolve")
    # masked route vs numpy rfft/irfft + direct circular sum
    for kind in ("band", "random"):
        if kind == "band":
            mask = np.zeros((H, 128), np.uint8)
            mask[:, :27] = 1
        else:
            mask = (rng.random((H, 128)) < 0.5).astype(np.uint8)
        G = N // 128
        blk = np.minimum(np.arange(N + 1) // G, 127)
        mref = np.empty((B, H, N))
        kps = []
        for h in range(H):
            K = np.fft.rfft(np.concatenate([k[h], np.zeros(2 * N - L)])) * mask[h, blk]
            kp = np.fft.irfft(K, n=2 * N)
            kps.append(kp)
            idx = (np.arange(N)[:, None] - np.arange(2 * N)[None, :]) % (2 * N)
            for b in range(B):
                xx = np.concatenate([u[b, h] * w[b, h], np.zeros(N)])
                mref[b, h] = (kp[None, :] * xx[idx]).sum(1) * v[b, h]
        if rel(oracle.fft_conv(u, k, w, v, mask=mask, lib=lib), mref) > 1e-12:
            failed.append(f"mask_{kind}")
        kp_o = oracle.masked_filter(k[1], N, mask[1], lib=lib)
        if rel(kp_o, kps[1]) > 1e-12:
            failed.append(f"masked_filter_{kind}")
    return failed


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_oracle_passes_compact_pins(mutant_dir):
    out = os.path.join(str(mutant_dir), "orig.so")
    oracle.build(out=out)
    assert _pins_hold(oracle.load(out)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_dir):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = os.path.join(str(mutant_dir), f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(str(mutant_dir), f"{name}.so")
    oracle.build(src=path, out=so)
    assert _pins_hold(oracle.load(so)) != [], f"mutant {name} passed every pin"
