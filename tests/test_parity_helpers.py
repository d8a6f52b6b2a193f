"""Host logic of the parity harness: the tolerance check must reject NaN and
infinities that the reference does not have, and accept equal infinities."""
import numpy as np
import pytest

from tests import parity


def test_within_tolerance_passes():
    ref = np.array([1.0, -2.0, 0.0, -np.inf])
    gpu = ref + np.array([0.005, -0.01, 0.0019, 0.0])
    assert parity.assert_close(gpu, ref) <= 0.0101


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, 1.02])
def test_mismatch_is_caught(bad):
    ref = np.array([1.0, 0.5])
    gpu = np.array([bad, 0.5])
    with pytest.raises(AssertionError):
        parity.assert_close(gpu, ref)


def test_nan_in_reference_position_is_caught():
    with pytest.raises(AssertionError):
        parity.assert_close(np.array([0.0]), np.array([np.nan]))
