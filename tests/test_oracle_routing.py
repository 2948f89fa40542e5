"""Pins of the oracle's routing and block alignment.

* top-k choice  -> brute force over every subset of top_k experts (the chosen
                   set is the one with the largest logit sum when logits are
                   distinct), and the lower-index rule on ties.
* router weights -> sum to one; ratios equal exp(logit difference); with
                   top_k = E they equal the full softmax (scipy); E = 1 gives
                   exactly 1.
* alignment     -> Python's sorted() by (expert, slot) and the structural
                   invariants of the padded layout.
"""

import itertools

import numpy as np
import pytest
import scipy.special

from oracle import moe as O


def _distinct_logits(rng, M, E):
    # distinct values per row: a random permutation of spaced levels plus noise
    base = np.stack([rng.permutation(E) for _ in range(M)]).astype(np.float32)
    return (base * 0.37 + rng.uniform(-0.1, 0.1, size=(M, E))).astype(np.float32)


@pytest.mark.parametrize("E,top_k", [(4, 1), (4, 2), (6, 3), (8, 2), (5, 5)])
def test_topk_matches_subset_brute_force(E, top_k):
    rng = np.random.default_rng(E * 10 + top_k)
    lg = _distinct_logits(rng, 12, E)
    ids, _ = O.route_topk(lg, top_k)
    for t in range(lg.shape[0]):
        best = max(itertools.combinations(range(E), top_k),
                   key=lambda s: sum(float(lg[t, e]) for e in s))
        assert set(ids[t].tolist()) == set(best)
        # listed from the largest logit down
        assert all(lg[t, ids[t, j]] > lg[t, ids[t, j + 1]] for j in range(top_k - 1))


def test_topk_ties_take_lower_index():
    lg = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]], np.float32)
    ids, w = O.route_topk(lg, 2)
    assert ids.tolist() == [[1, 2]]
    assert w[0, 0] == w[0, 1] == np.float32(0.5)


@pytest.mark.parametrize("E,top_k", [(4, 3), (8, 2), (8, 5), (16, 8)])
def test_topk_ties_match_sorted_rows(E, top_k):
    """Small-integer logits (ties everywhere, tied values displaced down the
    list by larger ones): each row's choice equals Python's sorted() by
    (logit descending, expert ascending), cut at top_k."""
    rng = np.random.default_rng(100 + E + top_k)
    lg = rng.integers(0, 4, size=(400, E)).astype(np.float32)
    lg[0, :] = 0.0
    lg[0, :4] = [5, 3, 3, 4]
    ids, _ = O.route_topk(lg, top_k)
    for t in range(lg.shape[0]):
        want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:top_k]
        assert ids[t].tolist() == want
    if top_k == 3 and E == 4:
        assert ids[0].tolist() == [0, 3, 1]


def test_router_weights_sum_to_one_and_ratios():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((500, 8)).astype(np.float32)
    ids, w = O.route_topk(lg, 2)
    s = w.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(s - 1.0)) <= 2 * np.finfo(np.float32).eps
    l0 = np.take_along_axis(lg, ids[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(lg, ids[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w[:, 1] / w[:, 0], np.exp(l1 - l0), rtol=1e-6)
    assert np.all(w[:, 0] >= w[:, 1])


def test_router_weights_full_softmax_when_top_k_equals_E():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((50, 6)).astype(np.float32)
    ids, w = O.route_topk(lg, 6)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-6)


def test_single_expert_weight_is_exactly_one():
    lg = np.random.default_rng(5).standard_normal((17, 1)).astype(np.float32)
    ids, w = O.route_topk(lg, 1)
    assert np.all(ids == 0) and np.all(w == 1.0)


@pytest.mark.parametrize("M,E,top_k,bm", [(1, 4, 2, 16), (37, 8, 2, 16), (64, 8, 2, 128),
                                          (200, 5, 3, 32), (0, 8, 2, 16), (9, 16, 1, 64)])
def test_align_matches_sorted_and_invariants(M, E, top_k, bm):
    rng = np.random.default_rng(M + 100 * E)
    ids, _ = O.route_topk(rng.standard_normal((M, E)).astype(np.float32), top_k)
    sorted_ids, expert_ids, total = O.align_block_size(ids, E, bm)
    S = M * top_k
    flat = ids.reshape(-1)
    # Python sorted() by (expert, slot)
    want = sorted(range(S), key=lambda i: (int(flat[i]), i))
    got = [int(v) for v in sorted_ids[:total] if v != S]
    assert got == want
    # sizes and padding
    counts = np.bincount(flat, minlength=E) if S else np.zeros(E, int)
    assert total == sum(-(-int(c) // bm) * bm for c in counts)
    assert total % bm == 0
    assert sorted_ids.size == O.align_max_padded(M, E, top_k, bm)
    assert np.all(sorted_ids[total:] == S)
    # every block holds one expert, and the listed expert is that of its slots
    for b in range(total // bm):
        blk = sorted_ids[b * bm:(b + 1) * bm]
        real = blk[blk != S]
        assert real.size > 0
        assert np.all(flat[real] == expert_ids[b])
    assert np.all(expert_ids[total // bm:] == -1)
    assert np.all(np.diff(expert_ids[:total // bm]) >= 0)
