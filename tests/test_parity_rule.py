"""The GPU parity tests' comparison rule, on the CPU: a NaN on one side, an
infinity of the wrong sign or a value outside the tolerance fails; NaN on both
sides and equal infinities pass (a comparison with NaN is false, so the rule is
written as what passes)."""

import numpy as np
import pytest

from tests.gpu_util import assert_close

REF = np.array([1.0, -2.0, np.nan, np.inf, 0.0])


def test_values_within_tolerance_pass():
    max_abs, max_rel = assert_close(np.array([1.005, -2.0, np.nan, np.inf, 0.009]), REF, "bf16")
    assert max_abs == pytest.approx(0.009) and max_rel == pytest.approx(0.005)


@pytest.mark.parametrize("k,value", [(0, np.nan), (2, 0.0), (3, -np.inf), (3, 1e300),
                                     (1, -2.05), (4, 0.011)])
def test_planted_mismatches_fail(k, value):
    got = np.array([1.0, -2.0, np.nan, np.inf, 0.0])
    got[k] = value
    with pytest.raises(AssertionError):
        assert_close(got, REF, "bf16")
