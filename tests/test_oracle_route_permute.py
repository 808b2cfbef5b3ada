"""Pins of the oracle's router, histogram, scan, scatter and block map.

Checked against a second implementation written differently (Python's stable
sort on (-logit, index)), library routines (scipy softmax, numpy stable
argsort), hand cases and invariants that any correct counting sort satisfies.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_logits(r, T, E, ties=False):
    l = r.standard_normal((T, E)).astype(np.float32)
    if ties:
        # coarse values produce many exact ties, including +0 and -0
        l = np.round(l * 2).astype(np.float32) / 2
        l[r.random((T, E)) < 0.1] = -0.0
        l[r.random((T, E)) < 0.1] = 0.0
    return l


def _python_topk(row, k):
    # Python's sort is stable and compares -0.0 == 0.0
    return sorted(range(len(row)), key=lambda e: -float(row[e]))[:k]


@pytest.mark.parametrize("T,E,k,ties", [(64, 8, 2, False), (64, 8, 2, True), (32, 256, 8, True),
                                        (32, 256, 8, False), (16, 5, 5, True), (16, 7, 1, True)])
def test_route_matches_python_sort(T, E, k, ties):
    r = np.random.default_rng(T * 1000 + E + k + ties)
    l = _rand_logits(r, T, E, ties)
    ids, w = O.route(l, k)
    for t in range(T):
        assert list(ids[t]) == _python_topk(l[t], k)
        # weights = scipy softmax over the chosen logits = full softmax renormalised on the top k
        sel = l[t, ids[t]].astype(np.float64)
        assert np.allclose(w[t], softmax(sel), rtol=0, atol=1e-15)
        p = softmax(l[t].astype(np.float64))
        assert np.allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=0, atol=1e-14)
        assert abs(w[t].sum() - 1.0) < 1e-15


def test_route_hand_cases():
    ids, w = O.route(np.array([[1, 3, 3, 2]], np.float32), 2)
    assert list(ids[0]) == [1, 2] and np.allclose(w[0], [0.5, 0.5])
    # all equal -> the k lowest indices, weight 1/k exactly
    ids, w = O.route(np.full((3, 16), 0.25, np.float32), 4)
    assert (ids == np.arange(4)).all() and (w == 0.25).all()
    # k = 1 -> weight exactly 1
    ids, w = O.route(np.array([[0.1, -2.0, 5.0]], np.float32), 1)
    assert ids[0, 0] == 2 and w[0, 0] == 1.0
    # -0 and +0 tie: lower index first
    ids, _ = O.route(np.array([[-1.0, 0.0, -0.0, -3.0]], np.float32), 2)
    assert list(ids[0]) == [1, 2]
    ids, _ = O.route(np.array([[-1.0, -0.0, 0.0, -3.0]], np.float32), 2)
    assert list(ids[0]) == [1, 2]
    # -inf logits are never chosen while k finite ones exist
    ids, _ = O.route(np.array([[-np.inf, 1.0, -np.inf, 0.5]], np.float32), 2)
    assert list(ids[0]) == [1, 3]
    # descending order and two-term softmax in closed form
    ids, w = O.route(np.array([[0.0, 2.0, 1.0]], np.float32), 2)
    assert list(ids[0]) == [1, 2]
    assert np.isclose(w[0, 0], 1 / (1 + np.exp(-1.0)), rtol=0, atol=1e-16)


def test_route_rejects_nan_and_too_few_finite():
    with pytest.raises(AssertionError):
        O.route(np.array([[np.nan, 1.0, 2.0]], np.float32), 1)
    with pytest.raises(AssertionError):
        O.route(np.array([[-np.inf, -np.inf, 2.0]], np.float32), 2)


def _permutation(T, E, k, seed, ties=False):
    r = np.random.default_rng(seed)
    ids, _ = O.route(_rand_logits(r, T, E, ties), k)
    counts = O.histogram(ids, E)
    offsets = O.exclusive_scan(counts)
    st, row_of = O.scatter(ids, offsets)
    return ids, counts, offsets, st, row_of


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (200, 256, 8), (37, 5, 5), (1, 256, 8), (64, 3, 1)])
def test_permutation_invariants(T, E, k):
    ids, counts, offsets, st, row_of = _permutation(T, E, k, seed=T + E + k, ties=True)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) == counts).all()
    # row_of and sorted_token are a bijection onto [0, T*k) and agree with each other
    assert np.array_equal(np.sort(row_of), np.arange(T * k))
    assert (st[row_of] == np.repeat(np.arange(T), k)).all()
    # every row p lies in the segment of the expert its assignment chose
    for e in range(E):
        seg = np.arange(offsets[e], offsets[e + 1])
        tok = st[seg]
        assert (np.diff(tok) > 0).all()                 # ascending, one row per token
        assert all(e in ids[t] for t in tok)
    # equals numpy's stable argsort of the flattened expert ids
    order = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(st, (order // k).astype(np.int32))
    assert np.array_equal(row_of[order], np.arange(T * k))


def test_k_equals_E_gives_every_expert_every_token():
    ids, counts, offsets, st, row_of = _permutation(12, 6, 6, seed=1)
    assert (counts == 12).all()
    assert np.array_equal(st, np.tile(np.arange(12), 6))


def test_each_token_in_k_plus_one_rows():
    """8 routed + 1 shared expert per token: every token is in exactly k+1 permuted rows."""
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    E, k = facts["routed_experts"]["value"], facts["experts_selected"]["value"]
    T = 300
    ids, counts, offsets, st, row_of = _permutation(T, E, k, seed=2)
    tiles = O.block_map(counts, offsets, T, k, 32)
    rows_token = np.concatenate([st, np.arange(T)])       # shared rows T*k + t carry token t
    covered = np.zeros(T * k + T, np.int64)
    for g, a, b in tiles:
        covered[a:b] += 1
    assert (covered == 1).all()
    assert (np.bincount(rows_token, minlength=T) == k + facts["shared_experts"]["value"]).all()


@pytest.mark.parametrize("BM", [1, 16, 32, 64, 128, 256])
def test_block_map_brute_force(BM):
    T, E, k = 150, 16, 4
    ids, counts, offsets, st, row_of = _permutation(T, E, k, seed=BM)
    tiles = O.block_map(counts, offsets, T, k, BM)
    expect = []
    for g in range(E + 1):
        lo, hi = (offsets[g], offsets[g + 1]) if g < E else (T * k, T * k + T)
        p = lo
        while p < hi:
            expect.append((g, p, min(p + BM, hi)))
            p += BM
    assert [tuple(t) for t in tiles] == expect
    n = sum(-(-int(c) // BM) for c in counts) + -(-T // BM)
    assert len(tiles) == n
    assert ((tiles[:, 2] - tiles[:, 1] >= 1) & (tiles[:, 2] - tiles[:, 1] <= BM)).all()
    assert (np.diff(tiles[:, 0]) >= 0).all()


def test_block_map_skips_empty_groups():
    counts = np.array([0, 5, 0, 0, 3], np.int32)
    offsets = O.exclusive_scan(counts)
    tiles = O.block_map(counts, offsets, T=4, k=2, BM=4)
    assert [tuple(t) for t in tiles] == [(1, 0, 4), (1, 4, 5), (4, 5, 8), (5, 8, 12)]
