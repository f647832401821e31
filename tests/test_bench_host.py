"""Host-side logic of bench.py, on the CPU: the algorithmic bytes each workload's
roofline divides by (against the configuration table: activations read and
written once, the spectrum read once per channel, the masked blocks skipped),
the path labels, the backward call's byte count, and the refusal of more than
one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

bench = pytest.importorskip("bench")
from long_fft_convolution_amd import synth  # noqa: E402

W = synth.WORKLOADS


def test_forward_algorithmic_bytes():
    # C2: u, w, v read and out written in fp16 (8 B per element) + 768 spectra of 1025 bins x 4 B
    assert bench.algorithmic_bytes(W["gated_fp16_n1k"]) == 64 * 768 * 1024 * 8 + 768 * 1024 * 4
    # C3: bf16, gated; spectra of 16384 bins x 4 B
    assert bench.algorithmic_bytes(W["gated_bf16_n16k"]) == 4 * 2560 * 16384 * 8 + 2560 * 16384 * 4
    # C4: ungated fp16 (4 B per element)
    assert bench.algorithmic_bytes(W["ungated_fp16_n1m"]) == 256 * (1 << 20) * 4 + 256 * (1 << 20) * 4
    # C5: 27 of 128 mask blocks kept: that share of the spectrum is read
    n = 1 << 22
    assert bench.algorithmic_bytes(W["partial_sparse_n4m"]) == int(128 * n * 4 + 128 * n * 4 * 27 / 128)
    # the short-filter path reads the 2048-bin window spectrum per channel
    assert bench.algorithmic_bytes(W["short_fp16_n1m_l512"]) == 256 * (1 << 20) * 4 + 256 * 2048 * 4
    # the configuration table's figures (MB)
    for name, mb in (("gated_fp16_n1k", 405.8), ("gated_bf16_n16k", 1510.0), ("ungated_fp16_n1m", 2147.5),
                     ("partial_sparse_n4m", 2600.5)):
        assert abs(bench.algorithmic_bytes(W[name]) / 1e6 - mb) < 1.0, name


def test_backward_algorithmic_bytes():
    wl = W["gated_fp16_n1k"]
    e, elems = 2, 64 * 768 * 1024
    # gated: dy, u, w, v read; du, dw, dv written; dk written; the spectrum read
    assert bench.bwd_algorithmic_bytes(wl, True, True) == elems * e * 7 + 768 * 1024 * e + 768 * 1025 * 4
    # ungated short filter: dy, u read, du written
    ws = W["short_fp16_n1m_l512"]
    assert bench.bwd_algorithmic_bytes(ws, False, False) == 256 * (1 << 20) * 2 * 3 + 256 * 512 * 2 + 256 * 2048 * 4


def test_path_labels():
    assert bench.path_of(W["gated_fp16_n1k"])[0] == "pair1k_kernel"
    assert bench.path_of(W["gated_bf16_n16k"])[0] == "pair16k_kernel"
    assert bench.path_of(W["ungated_fp32_n1k"])[0] == "fused_conv_kernel"
    assert bench.path_of(W["ungated_fp16_n1m"])[0].startswith("mp_pass1+mp_pass2m+mp_pass3")
    assert bench.path_of(W["partial_sparse_n4m"])[0].startswith("mp_pass1c+mp_pass2m+mp_pass3c")
    assert "windows" in bench.path_of(W["short_fp16_n1m_l512"])[0]
    for name in ("gated_fp16_n1k", "gated_bf16_n16k", "ungated_fp16_n1m", "partial_sparse_n4m"):
        assert bench.path_of(W[name])[1] == "f16"
    assert bench.path_of(W["ungated_fp32_n1k"])[1] == "f32"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
