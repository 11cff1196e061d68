"""The CPU oracle against its pins (values printed on the pages, closed forms,
library routines, algebraic laws, brute force).  Runs without a GPU."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_oracle_threads_match_single_thread(oracle_lib):
    import numpy as np
    import workloads
    x = workloads.config(2, 0, 64)
    y1 = oracle_lib.softmax(x, threads=1)
    y4 = oracle_lib.softmax(x, threads=4)
    assert np.array_equal(y1, y4)
    p1, i1 = oracle_lib.topk(workloads.config(5, 0, 3), 8, threads=1)
    p3, i3 = oracle_lib.topk(workloads.config(5, 0, 3), 8, threads=3)
    assert np.array_equal(p1, p3) and np.array_equal(i1, i3)
