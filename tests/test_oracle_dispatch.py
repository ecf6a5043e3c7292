"""Pins for the oracle's dispatch step (oracle.moe.dispatch).

Contract: ruDNN user guide (RUDA docs), section 5: dispatch drops no token
for a capacity limit, the order inside an expert is not fixed, and a stored
mapping restores token order; the experts page (docs.rs ruDNN 0.1.25,
src/moe/experts.rs, forward_dispatched_with_strategy) relies on complete,
monotone expert segments.
Pins: numpy.bincount / cumsum for counts and offsets, a bijection check on
the stored mapping, and a brute-force scan of the routing table for the
token set of every expert.
"""

import numpy as np
import pytest

from oracle.moe import dispatch


def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(
        np.uint32) if T else np.zeros((0, k), np.uint32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 2), (17, 8, 8),
                                   (64, 16, 4), (0, 4, 2), (33, 64, 1)])
def test_dispatch_invariants(T, E, k):
    rng = np.random.default_rng(T * 100 + E * 10 + k)
    idx = _random_idx(rng, T, E, k)
    x = rng.integers(0, 2 ** 16, size=(T, 6)).astype(np.uint16)
    d = dispatch(x, idx, E)
    N = T * k
    np.testing.assert_array_equal(
        d["counts"], np.bincount(idx.ravel().astype(np.int64), minlength=E))
    np.testing.assert_array_equal(d["offsets"][1:], np.cumsum(d["counts"]))
    assert d["offsets"][0] == 0 and d["offsets"][E] == N      # no drops
    assert np.all(np.diff(d["offsets"]) >= 0)                  # monotone
    tr = d["token_row"].ravel()
    assert sorted(tr.tolist()) == list(range(N))               # bijection
    for t in range(T):
        for j in range(k):
            r = int(d["token_row"][t, j])
            assert d["row_expert"][r] == idx[t, j]
            assert d["row_token"][r] == t
            np.testing.assert_array_equal(d["xd"][r], x[t])    # bit copy
    for e in range(E):
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        assert np.all(d["row_expert"][lo:hi] == e)
        brute = sorted(t for t in range(T) for j in range(k) if idx[t, j] == e)
        assert sorted(d["row_token"][lo:hi].tolist()) == brute


def test_dispatch_is_stable():
    idx = np.array([[2, 0], [0, 1], [2, 1], [0, 2]], dtype=np.uint32)
    d = dispatch(np.zeros((4, 1)), idx, 3)
    assert d["offsets"].tolist() == [0, 3, 5, 8]
    assert d["row_token"].tolist() == [0, 1, 3, 1, 2, 0, 2, 3]
    assert d["token_row"].tolist() == [[5, 0], [1, 3], [6, 4], [2, 7]]
