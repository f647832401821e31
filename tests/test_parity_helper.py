"""Pins for the comparison functions every GPU parity test goes through
(oracle.rel_l2, oracle.seq_rel_l2, oracle.max_abs and tests/parity.check),
on the CPU: hand-computed values, and a planted wrong sequence that the
whole-tensor error alone would let through."""
import numpy as np
import pytest

import oracle
from parity import check, metrics


def test_rel_l2_hand_values():
    # ||(1,2) - (1,0)|| / ||(1,0)|| = ||(0,2)|| / 1 = 2
    assert oracle.rel_l2([1.0, 2.0], [1.0, 0.0]) == 2.0
    # ||(3,4)|| / ||(0,5)|| = 5 / 5 = 1  (a = (3, 9), b = (0, 5))
    assert oracle.rel_l2([3.0, 9.0], [0.0, 5.0]) == 1.0
    assert oracle.rel_l2([1.5, -2.0, 7.0], [1.5, -2.0, 7.0]) == 0.0
    # an all-zero reference: the absolute norm
    assert oracle.rel_l2([3.0, 4.0], [0.0, 0.0]) == 5.0


def test_seq_rel_l2_hand_values():
    a = np.array([[[1.0, 2.0], [3.0, 4.0]], [[0.0, 0.0], [6.0, 8.0]]])
    b = np.array([[[1.0, 0.0], [3.0, 0.0]], [[0.0, 0.0], [6.0, 8.0]]])
    # sequences (0,0): 2/1; (0,1): 4/3; (1,0): zero reference, zero error; (1,1): exact
    np.testing.assert_array_equal(oracle.seq_rel_l2(a, b), [2.0, 4.0 / 3.0, 0.0, 0.0])
    assert oracle.seq_rel_l2([3.0, 9.0], [0.0, 5.0]).tolist() == [1.0]
    with pytest.raises(ValueError):
        oracle.seq_rel_l2(np.zeros((2, 3)), np.zeros((3, 2)))


def test_max_abs_hand_values():
    assert oracle.max_abs([1.0, -5.0, 2.0], [1.5, 2.0, 2.0]) == 7.0
    assert oracle.max_abs(np.zeros((2, 0)), np.zeros((2, 0))) == 0.0


def test_check_accepts_close_results():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 4, 256))
    got = ref * (1 + 1e-4 * rng.standard_normal(ref.shape))
    m = check(got, ref, 5e-3, "close")
    assert m["n_seq"] == 12 and m["rel_l2"] < 2e-4 and m["worst_seq_rel_l2"] < 3e-4


def test_check_rejects_one_wrong_sequence_among_many():
    # 49,152 sequences (the N = 1024 gated workload's B * H); one of them zeroed
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((64, 768, 16))
    got = ref * (1 + 1e-4 * rng.standard_normal(ref.shape))
    got[17, 300, :] = 0.0
    m = metrics(got, ref)
    # the whole-tensor error alone passes the fp16 bound ...
    assert m["rel_l2"] < 5e-3
    # ... the per-sequence bound does not, and names the sequence
    assert m["worst_seq"] == 17 * 768 + 300
    with pytest.raises(AssertionError, match="sequence 13356"):
        check(got, ref, 5e-3, "planted")


def test_check_rejects_non_finite_and_shape_mismatch():
    ref = np.ones((2, 8))
    got = ref.copy()
    got[1, 3] = np.inf
    with pytest.raises(AssertionError, match="non-finite"):
        check(got, ref, 1.0, "inf")
    with pytest.raises(AssertionError, match="shape"):
        check(np.ones((2, 7)), ref, 1.0, "shape")
