"""Pins of the oracle's pooled block scores and hybrid Top-k / Top-p selection
(Prism guide (pt), Método 3).  CPU only."""

import itertools
import math

import numpy as np
import pytest

import oracle as O


def _rand_row(rng, nb, spread=2.0):
    s = rng.standard_normal(nb) * spread
    sizes = rng.choice([64, 128, 256], nb)
    return s, O.block_probabilities(s), sizes


def test_softmax_rows():
    rng = np.random.default_rng(0)
    s = rng.standard_normal((5, 9)) * 3
    P = O.block_probabilities(s)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-15)
    import torch
    np.testing.assert_allclose(P, torch.softmax(torch.tensor(s), dim=1).numpy(), rtol=1e-14)


def test_pooling_is_block_mean():
    rng = np.random.default_rng(1)
    blk_start = np.array([0, 1, 3, 4, 8])
    x = rng.standard_normal((512, 4))
    pooled = O.pool_blocks(x, blk_start)
    for b in range(4):
        np.testing.assert_allclose(pooled[b], x[blk_start[b] * 64:blk_start[b + 1] * 64].mean(0), rtol=1e-14)


def test_full_selection_cases():
    rng = np.random.default_rng(2)
    s, P, sizes = _rand_row(rng, 40)
    assert O.select_row(s, P, sizes, 2, 1.0, 1.0, 10 ** 6)["L"] == 40          # p = 1
    assert O.select_row(s, P, sizes, 40, 0.1, 1.0, 10 ** 6)["L"] == 40         # k >= n_b
    assert O.select_row(s, P, sizes, 99, 0.1, 1.0, 10 ** 6)["L"] == 40
    r = O.select_row(s, P, sizes, 1, 1e-12, 1.0, 10 ** 6)                      # tiny p: Top-1 only
    assert r["L"] == 1 and r["cols"][0] == int(np.argmax(s))


def test_union_of_topk_and_topp():
    """Without a cap, S_i equals the literal union of the Top-k set and the
    Top-p (nucleus) set computed separately."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        nb = int(rng.integers(2, 60))
        s, P, sizes = _rand_row(rng, nb, spread=float(rng.uniform(0.1, 4)))
        k = int(rng.integers(1, 8))
        p = float(rng.uniform(0.05, 0.99))
        topk = set(np.argsort(-s, kind="stable")[:k].tolist())
        nucleus, mass = set(), 0.0
        for j in sorted(range(nb), key=lambda j: (-P[j], j)):
            if mass >= p:
                break
            nucleus.add(j)
            mass += P[j]
        got = O.select_row(s, P, sizes, k, p, 1.0, 10 ** 9)
        assert set(got["cols"].tolist()) == topk | nucleus, trial


def _brute_force(s, P, sizes, k, p, cap, N):
    """Enumerate all subsets: keep those closed upwards in the (score desc,
    index asc) order; among them the smallest one that holds the Top-k floor
    and, unless that would exceed the token budget, reaches mass p."""
    nb = s.size
    rank = {j: r for r, j in enumerate(sorted(range(nb), key=lambda j: (-s[j], j)))}
    closed = []
    for bits in range(1, 1 << nb):
        S = [j for j in range(nb) if bits >> j & 1]
        if max(rank[j] for j in S) == len(S) - 1:
            closed.append(S)
    closed.sort(key=len)
    n_k = min(k, nb)
    U = math.floor(cap * N) if cap < 1 else math.inf
    reach = [S for S in closed if P[S].sum() >= p] if p < 1 else [closed[-1]]
    nucleus = reach[0] if reach else closed[-1]
    fits = [S for S in closed if sizes[S].sum() <= U]
    longest_fit = len(fits[-1]) if fits else 0
    L = max(n_k, min(len(nucleus), longest_fit))
    return sorted(next(S for S in closed if len(S) == L))


def test_brute_force_small_rows():
    rng = np.random.default_rng(4)
    for trial in range(150):
        nb = int(rng.integers(1, 11))
        s, P, sizes = _rand_row(rng, nb, spread=float(rng.uniform(0.2, 3)))
        k = int(rng.integers(1, 5))
        p = float(rng.choice([0.3, 0.6, 0.9, 0.97, 1.0]))
        cap = float(rng.choice([1.0, 0.5, 0.2, 0.05]))
        N = 2048
        got = O.select_row(s, P, sizes, k, p, cap, N)
        assert got["cols"].tolist() == _brute_force(s, P, sizes, k, p, cap, N), trial


def test_selection_invariants():
    rng = np.random.default_rng(5)
    N = 10 ** 5
    for trial in range(100):
        nb = int(rng.integers(5, 300))
        s, P, sizes = _rand_row(rng, nb, spread=float(rng.uniform(0.05, 3)))
        k, p, cap = int(rng.integers(1, 20)), float(rng.uniform(0.2, 0.99)), float(rng.choice([1.0, 0.1, 0.02]))
        r = O.select_row(s, P, sizes, k, p, cap, N)
        cols = r["cols"]
        assert cols.size >= min(k, nb)
        assert (np.diff(cols) > 0).all()
        outside = np.setdiff1d(np.arange(nb), cols)
        if outside.size:
            assert s[outside].max() <= s[cols].min()                      # a prefix of the score order
        capped = sizes[cols].sum() > math.floor(cap * N) if cap < 1 else False
        if P[cols].sum() < p - 1e-12:                                     # short of p only when the cap bound
            assert cap < 1
            nxt = r["order"][cols.size]
            assert capped or sizes[cols].sum() + sizes[nxt] > math.floor(cap * N)
        if capped:                                                        # over budget only from the Top-k floor
            assert cols.size == min(k, nb)


def test_csr_and_transpose():
    rng = np.random.default_rng(6)
    nb = 23
    rows = [np.sort(rng.choice(nb, int(rng.integers(1, nb)), replace=False)) for _ in range(nb)]
    ptr, col = O.csr_from_rows(rows)
    tptr, tcol = O.csr_transpose(ptr, col, nb)
    dense = np.zeros((nb, nb), bool)
    for i, r in enumerate(rows):
        dense[i, r] = True
    for j in range(nb):
        assert tcol[tptr[j]:tptr[j + 1]].tolist() == np.nonzero(dense[:, j])[0].tolist()


def test_tie_detection():
    s = np.array([3.0, 2.0, 2.0 + 5e-7, 1.0, 0.0])
    P = O.block_probabilities(s)
    sizes = np.full(5, 64)
    sel = O.select_row(s, P, sizes, 2, 0.5, 1.0, 10 ** 6)
    assert sel["L"] == 2 and O.row_tie_affected(s, sel, 0.5, False)
    # the other member of the tie is a valid alternative; a gap is not
    assert O.row_is_valid_alternative(s, np.array([0, 1]), sel)
    assert O.row_is_valid_alternative(s, np.array([0, 2]), sel)
    assert not O.row_is_valid_alternative(s, np.array([0, 3]), sel)
    sel2 = O.select_row(np.array([3.0, 2.0, 1.0]), O.block_probabilities(np.array([3.0, 2.0, 1.0])),
                        np.full(3, 64), 1, 0.5, 1.0, 10 ** 6)
    assert not O.row_tie_affected(np.array([3.0, 2.0, 1.0]), sel2, 0.5, False)
