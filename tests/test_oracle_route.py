"""Pins of the oracle's route pack (CPU only)."""

import numpy as np
import pytest

from oracle import route


def _library_pack(ids, w, E):
    flat = ids.reshape(-1)
    keep = (flat >= 0) & (flat < E)
    q = np.nonzero(keep)[0]
    order = q[np.argsort(flat[q], kind="stable")]
    count = np.bincount(flat[q], minlength=E)
    offset = np.concatenate([[0], np.cumsum(count)])
    return count, offset, order, w.reshape(-1)[order]


@pytest.mark.parametrize("rows,topk,E,seed", [(16, 2, 8, 0), (33, 8, 128, 1),
                                               (1, 8, 192, 2), (200, 4, 5, 3)])
def test_matches_stable_argsort(rows, topk, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(rows, topk))
    w = rng.random((rows, topk))
    got = route.route_pack(ids, w, E)
    count, offset, order, wo = _library_pack(ids, w, E)
    n = len(order)
    assert np.array_equal(got["count"], count)
    assert np.array_equal(got["offset"], offset)
    assert np.array_equal(got["pair_of_pos"][:n], order)
    assert np.all(got["pair_of_pos"][n:] == -1)
    assert np.array_equal(got["weight_of_pos"][:n], wo)
    assert got["num_active"] == int(np.count_nonzero(count))
    inv = np.full(rows * topk, -1)
    inv[order] = np.arange(n)
    assert np.array_equal(got["pos_of_pair"], inv)


def test_drops_out_of_range_and_keeps_duplicates():
    ids = np.array([[0, 0], [5, -1], [2, 9], [2, 2]])
    w = np.arange(8, dtype=float).reshape(4, 2)
    got = route.route_pack(ids, w, 3)
    assert got["dropped"] == 3
    assert list(got["count"]) == [2, 0, 3]
    assert list(got["pair_of_pos"][:5]) == [0, 1, 4, 6, 7]
    assert list(got["pos_of_pair"]) == [0, 1, -1, -1, 2, -1, 3, 4]
    assert got["num_active"] == 2


def test_stability_within_expert():
    ids = np.full((10, 1), 3)
    got = route.route_pack(ids, np.ones((10, 1)), 4)
    assert list(got["pair_of_pos"][:10]) == list(range(10))
