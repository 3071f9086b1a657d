"""Pins of the oracle's block Top-k (first paragraph of the MicroAdam page:
(I_t, V_t) = T_k(|a_t|)) against a full sort, brute force over subsets, and
the q-contraction of the third paragraph."""
import itertools

import numpy as np
import pytest

import oracle as O


def _key(a):
    return a.astype(np.float32).view(np.uint32) & np.uint32(0x7fffffff)


def _sort_reference(a, kb):
    key = _key(a).astype(np.int64)
    order = np.lexsort((np.arange(a.size), -key))   # key desc, position asc
    return np.sort(order[:kb])


@pytest.mark.parametrize("n,kb", [(1, 0), (1, 1), (7, 3), (64, 1), (100, 37), (16384, 164),
                                  (16384, 0), (16384, 16384), (11776, 118)])
def test_topk_equals_full_sort(n, kb):
    rng = np.random.default_rng(n * 131 + kb)
    a = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    a[rng.random(n) < 0.01] *= 50
    np.testing.assert_array_equal(O.topk(a, kb), _sort_reference(a, kb))


def test_topk_ties_go_to_lower_index():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 200))
        kb = int(rng.integers(0, n + 1))
        vals = np.array([0.0, -0.0, 1.0, -1.0, 2.5, -2.5, 1e-30, -1e-30], np.float32)
        a = vals[rng.integers(0, vals.size, n)]
        got = O.topk(a, kb)
        np.testing.assert_array_equal(got, _sort_reference(a, kb))
        if kb:
            # +1 and -1 have the same key, as do +0 and -0
            assert len(set(got.tolist())) == kb


def test_topk_brute_force_small():
    # the selected set S is the unique kb-subset in which every member outranks
    # every non-member under (|a| desc, index asc)
    rng = np.random.default_rng(6)
    for n in range(1, 9):
        for trial in range(6):
            a = rng.choice(np.array([0.0, 1.0, -1.0, 2.0, 3.0, -3.0], np.float32), n)
            key = _key(a)
            for kb in range(n + 1):
                winners = []
                for S in itertools.combinations(range(n), kb):
                    rest = [i for i in range(n) if i not in S]
                    if all((key[i] > key[r]) or (key[i] == key[r] and i < r) for i in S for r in rest):
                        winners.append(S)
                assert len(winners) == 1
                np.testing.assert_array_equal(O.topk(a, kb), np.array(winners[0], np.int32))


def test_topk_q_contraction():
    # ||a - T_k(a)||^2 <= (1 - k/n) ||a||^2 for magnitude Top-k (third paragraph,
    # q = sqrt(1 - k/d)), checked in double on the selected set
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(2, 5000))
        kb = int(rng.integers(0, n + 1))
        a = rng.standard_t(3, n).astype(np.float32)
        sel = O.topk(a, kb)
        r = a.astype(np.float64).copy()
        r[sel] = 0
        lhs = (r ** 2).sum()
        rhs = (1 - kb / n) * (a.astype(np.float64) ** 2).sum()
        assert lhs <= rhs * (1 + 1e-12) + 1e-300
