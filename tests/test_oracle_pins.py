"""The float64 oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_is_thread_count_independent(orc):
    import numpy as np
    import qmx_inputs as qi
    c = qi.affine_case(3, 64, 1024, 4, 64, qi.BF16, seed=12)
    n0 = orc.num_threads()
    try:
        orc.set_num_threads(1)
        a = orc.affine_case(c)
        orc.set_num_threads(max(2, n0))
        b = orc.affine_case(c)
    finally:
        orc.set_num_threads(n0)
    assert np.array_equal(a, b)
