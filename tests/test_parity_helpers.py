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


def test_selection_report_counts(oracle_lib):
    """The counting form of the selection rule: identical ids count nothing, an id outside the band
    is an exact mismatch, a different choice among tied blocks is an in-band flip."""
    from block_sparse_gqa_amd import synth
    oracle = oracle_lib
    inp = synth.custom((256,), (256,), 4, 2, 64, 32, 64, 2, seed=3, name="report")
    rows = np.arange(256, dtype=np.int64)
    ids, kth, tie = oracle.index_topk(inp, rows)
    rep = parity.selection_report(oracle, inp, rows, ids, ids, kth, tie)
    assert rep == dict(rows=256, pairs=512, near_tie=int(tie.sum()), exact_mismatch=0, band_flips=0)
    wrong = ids.copy()
    r = 255                                          # E = 4 > k = 2: the dropped blocks score lower
    dropped = sorted(set(range(4)) - set(ids[r, 0].tolist()))
    wrong[r, 0] = sorted([ids[r, 0, 0], dropped[0]])
    t2 = tie.copy()
    t2[r, 0] = False
    assert parity.selection_report(oracle, inp, rows, wrong, ids, kth, t2)["exact_mismatch"] == 1
    # all block scores equal: every row with E > k is a near tie, and any k blocks are inside the band
    inp.k_idx = synth.f32_to_bf16_bits(np.full(inp.k_idx.shape, 0.25, np.float32))
    ids, kth, tie = oracle.index_topk(inp, rows)
    assert tie[255].all()
    alt = ids.copy()
    alt[255, :] = [2, 3]
    rep = parity.selection_report(oracle, inp, rows, alt, ids, kth, tie)
    assert rep["band_flips"] == 2 and rep["exact_mismatch"] == 0
    # the invariants still hold inside the band: a duplicate is a mismatch
    alt[255, 0] = [3, 3]
    assert parity.selection_report(oracle, inp, rows, alt, ids, kth, tie)["exact_mismatch"] == 1
