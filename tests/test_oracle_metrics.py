import numpy as np

from oracle import metrics as Mx


def test_rel_l2_and_row_ratio_hand_values():
    ref = np.array([[3.0, 4.0], [0.0, 1.0]])
    y = np.array([[3.0, 4.0], [0.0, 1.0]])
    assert Mx.rel_l2(y, ref) == 0.0
    y2 = ref.copy()
    y2[0, 0] += 0.004                    # |ref| = sqrt(26); err = 0.004
    assert abs(Mx.rel_l2(y2, ref) - 0.004 / np.sqrt(26)) < 1e-15
    assert abs(Mx.row_maxabs_ratio(y2, ref) - 0.004 / 4.0) < 1e-15
    ok, rl, rr = Mx.check_output(y2, ref)
    assert ok
    y3 = ref.copy()
    y3[1, 0] = 0.05                      # row 1: 0.05 / 1.0 > 2e-2
    ok, rl, rr = Mx.check_output(y3, ref)
    assert not ok and rr == 0.05


def test_nonfinite_fails():
    ref = np.ones((2, 2))
    y = ref.copy()
    y[0, 0] = np.nan
    assert not Mx.check_output(y, ref)[0]
