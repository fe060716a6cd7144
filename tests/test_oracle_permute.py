"""Pins of the oracle's permutation (no GPU): a lexsort brute force and the
invariants of an expert-sorted pair list with expert-parallel rebase."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _brute(ids, E, off, E_loc, shared):
    T, k = ids.shape
    p = np.arange(T * k)
    e = ids.reshape(-1) - off
    ok = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < E) & (e >= 0) & (e < E_loc)
    keys_e = list(e[ok]) + ([E_loc] * T if shared else [])
    keys_p = list(p[ok]) + ([T * k + t for t in range(T)] if shared else [])
    order = np.lexsort((np.array(keys_p), np.array(keys_e))) if keys_p else []
    return np.array(keys_p, dtype=np.int64)[order] if keys_p else np.zeros(0, np.int64)


@pytest.mark.parametrize("T,k,E,off,E_loc,shared", [
    (37, 8, 256, 96, 32, 0), (64, 8, 288, 0, 288, 1), (1, 4, 128, 0, 128, 0),
    (300, 2, 8, 4, 4, 0), (0, 8, 64, 0, 64, 0), (5, 8, 256, 200, 56, 1)])
def test_permute_matches_lexsort_and_invariants(T, k, E, off, E_loc, shared):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else \
        np.zeros((0, k), np.int64)
    offsets, sp, pr, err = O.permute(ids, E, off, E_loc, shared)
    G = E_loc + shared
    assert err == 0
    assert offsets[0] == 0 and offsets[-1] == len(sp) and len(offsets) == G + 1
    assert np.array_equal(sp, _brute(ids, E, off, E_loc, shared))
    # counts are the bincount of local ids
    e = ids.reshape(-1) - off
    cnt = np.bincount(e[(e >= 0) & (e < E_loc)], minlength=E_loc)
    assert np.array_equal(np.diff(offsets)[:E_loc], cnt)
    # every local pair exactly once; pair_row inverts sorted_pair
    assert len(set(sp.tolist())) == len(sp)
    assert np.array_equal(pr[sp], np.arange(len(sp)))
    assert np.sum(pr >= 0) == len(sp)
    for p in range(T * k):
        local = 0 <= ids.reshape(-1)[p] - off < E_loc
        assert (pr[p] >= 0) == local


def test_permute_out_of_range_ids_set_error_and_are_skipped():
    ids = np.array([[3, 300], [-1, 5], [7, 2]])
    offsets, sp, pr, err = O.permute(ids, 256, 0, 256, 0)
    assert err == O.ERR_GLOBAL_ID_OOB
    assert sorted(sp.tolist()) == [0, 3, 4, 5]
    assert pr[1] == -1 and pr[2] == -1
