"""CPU test of the greedy-token check the decode parity tests use."""
import numpy as np

from greedy import greedy_ok


def test_clear_gap_requires_the_argmax_and_near_ties_accept_any_of_them():
    lg = np.array([4.79, 4.776, 4.756, 4.33, -1.0])   # max |logit| 4.79
    # tolerance 2e-2: margin 0.19; the top-2 gap 0.014 is not clear
    assert greedy_ok(0, lg, 2e-2) and greedy_ok(1, lg, 2e-2) and greedy_ok(2, lg, 2e-2)
    assert not greedy_ok(3, lg, 2e-2) and not greedy_ok(4, lg, 2e-2)
    # tolerance 1e-4: margin 9.6e-4 < gap, so only the argmax
    assert greedy_ok(0, lg, 1e-4) and not greedy_ok(1, lg, 1e-4)
    # a clear gap at any tolerance
    lg2 = np.array([0.0, 3.0, 1.0])
    assert greedy_ok(1, lg2, 2e-2) and not greedy_ok(2, lg2, 2e-2)
