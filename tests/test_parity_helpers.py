"""CPU checks of the comparison rules used by the GPU parity tests."""
import numpy as np

from tests import parity as P


def test_valid_sets_near_tie():
    l = np.array([3.0, 1.0, 0.9995, 0.5, 2.0])
    assert P.valid_sets(l, 2) == [(0, 4)]
    assert P.valid_sets(l, 3) == [(0, 1, 4), (0, 2, 4)]
    assert P.valid_sets(np.zeros(4), 2) == [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    assert P.valid_sets(l, 5) == [(0, 1, 2, 3, 4)]


def test_routing_report_flags_wrong_and_accepts_ties():
    logits = np.array([[3.0, 2.0, 0.0, -1.0],      # clear
                       [1.0, 0.5, 0.4999, 0.0],    # near tie for 2nd
                       [1.0, 0.9, 0.0, 0.1]])      # clear, slot order matters
    oidx = np.array([[0, 1], [0, 1], [0, 1]], np.int32)
    og = np.array([[0.7, 0.3], [0.6, 0.4], [0.52, 0.48]])
    ok = P.routing_report(np.array([[0, 1], [0, 2], [0, 1]]), og, logits, oidx, og, 2)
    assert ok["bad"] == [] and ok["near_ties"] == 1
    badset = P.routing_report(np.array([[0, 2], [0, 1], [0, 1]]), og, logits, oidx, og, 2)
    assert badset["bad"] == [0]
    badorder = P.routing_report(np.array([[0, 1], [0, 1], [1, 0]]), og, logits, oidx, og, 2)
    assert badorder["bad"] == [2]
    badtie = P.routing_report(np.array([[0, 1], [0, 3], [0, 1]]), og, logits, oidx, og, 2)
    assert badtie["bad"] == [1]


def test_rel_l2():
    a = np.ones((3, 4))
    assert P.rel_l2(a, a) == 0.0
    assert abs(P.rel_l2(a * 1.01, a) - 0.01) < 1e-12


def test_row_errors_catch_one_misplaced_row_among_many():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((100000, 64))
    got = ref * (1 + 2.0**-8 * rng.standard_normal(ref.shape))  # bf16-sized noise
    assert P.rel_l2(got, ref) < P.TOL_BF16
    assert P.row_errors(got, ref).max() < P.ROW_TOL_BF16
    got[[17, 18]] = got[[18, 17]]  # two tokens' rows swapped
    assert P.rel_l2(got, ref) < P.TOL_BF16  # the whole-output bound misses it
    err = P.row_errors(got, ref)
    assert err[17] > 10 * P.ROW_TOL_BF16 and err[18] > 10 * P.ROW_TOL_BF16
    # a row whose own norm is tiny is measured against the median row norm
    ref[3] *= 1e-6
    got[3] = ref[3] + 1e-9
    assert P.row_errors(got, ref)[3] < 1e-6
