"""The comparison rules of tests/parity.py, checked on the CPU with planted
mistakes: a selection that returns an id outside the candidate range (a
negative id would otherwise index a score array from its end), an id that is
not a candidate, a swap outside the tie band, a wrong count or padding, and
an attention output off by more than the tolerance all fail; accepted tie
swaps pass."""
import numpy as np
import pytest

from tests.parity import check_attention, check_pool, check_selection, check_topk


def _ranked(scores, k):
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))[:k]
    out = np.full(k, -1, np.int64)
    out[:len(order)] = sorted(order)
    return out, len(order)


def test_selection_accepts_exact_and_tie_swaps():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-7, 1.0, 0.5])
    ids, n = _ranked(s, 3)                   # {0, 1, 3}
    assert check_selection(ids, n, ids, n, lambda j: s[j], valid=len(s)) == 0
    swapped = np.array([0, 1, 2])            # 2 for 3: within 1e-5 of the 3rd score
    assert check_selection(swapped, 3, ids, n, lambda j: s[j], valid=len(s)) == 1


@pytest.mark.parametrize("bad", [[-1, 0, 1], [0, 1, 6], [0, 1, 4]])
def test_selection_rejects_out_of_range_and_non_ties(bad):
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-7, 1.0, 0.5])
    ids, n = _ranked(s, 3)
    with pytest.raises(AssertionError):
        check_selection(np.array(bad), 3, ids, n, lambda j: s[j % len(s)], valid=len(s))


def test_selection_rejects_non_candidates_count_and_padding():
    cand = np.array([10, 11, 12, 20, 21])
    sc = {10: 1.0, 11: 2.0, 12: 3.0, 20: 4.0, 21: 5.0}
    ref = {"cand": cand, "cand_scores": np.array([sc[j] for j in cand]),
           "topk": np.array([12, 20, 21, -1]), "n_topk": 3}
    assert check_topk(np.array([12, 20, 21, -1]), 3, ref) == 0
    for bad, n in (([13, 20, 21, -1], 3),       # 13 is no candidate
                   ([12, 20, 21, 11], 3),       # padding
                   ([12, 20, -1, -1], 2),       # count
                   ([20, 12, 21, -1], 3),       # order
                   ([12, 20, 21, -1], 9)):      # count past the list
        with pytest.raises(AssertionError):
            check_topk(np.array(bad), n, ref)


def test_pool_ids_must_be_visible_blocks():
    bs = np.array([1.0, 9.0, 3.0, 7.0])
    ref = {"block_scores": bs, "pool": np.array([1, 3])}
    assert check_pool(np.array([1, 3, -1]), 2, ref) == 0
    with pytest.raises(AssertionError):
        check_pool(np.array([-3, 1, -1]), 2, ref)        # bs[-3] would read block 1
    with pytest.raises(AssertionError):
        check_pool(np.array([1, 4, -1]), 2, ref)


def test_attention_tolerance_and_empty_rows():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 512))
    lse = np.array([1.0, -np.inf, 2.0])
    ref[1] = 0.0
    assert check_attention(ref * (1 + 1e-4), lse, ref, lse) <= 2e-3
    off = ref.copy()
    off[2, 7] += 3e-3 * np.abs(ref[2]).max()
    with pytest.raises(AssertionError):
        check_attention(off, lse, ref, lse)
    nan = ref.copy()
    nan[0, 0] = np.nan
    with pytest.raises(AssertionError):
        check_attention(nan, lse, ref, lse)
    with pytest.raises(AssertionError):
        check_attention(ref, np.array([1.0, 0.0, 2.0]), ref, lse)
