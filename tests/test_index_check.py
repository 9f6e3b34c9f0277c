"""prism_check_index on host arrays (no GPU): an index the oracle builds for
the method passes; every kind of malformed index is rejected, and `bad`
names where."""

import ctypes

import numpy as np
import pytest

import oracle as O
from dynamic_block_sparse_macro_amd import binding as B
from workload import generate


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        from dynamic_block_sparse_macro_amd.build import build
        build(verbose=False)
    return B.load_library()


def _index(name):
    """The oracle's index of every head of a workload, in the layout the
    library writes (row pointers over all heads, tails repeated)."""
    w = generate(name)
    c = w.cfg
    P = O.Params(top_k=c.top_k, top_p=c.top_p, density_cap=c.density_cap)
    res = O.run_pipeline(w.f32("q"), w.f32("k"), w.f32("v"), w.a, c.T, c.H, c.W, P, attention=False)
    tiles = c.N // 64
    heads = c.heads
    perm = np.zeros((heads, c.N), np.int32)
    bs = np.full((heads, tiles + 1), tiles, np.int32)
    nb = np.zeros(heads, np.int32)
    rp = np.zeros((heads, tiles + 1), np.int32)
    trp = np.zeros((heads, tiles + 1), np.int32)
    cols, tcols = [], []
    base = 0
    for h, hr in enumerate(res["heads"]):
        n = hr["n_blocks"]
        perm[h] = hr["perm"]
        bs[h, :n + 1] = hr["blk_start"]
        nb[h] = n
        rp[h, :n + 1] = hr["row_ptr"] + base
        rp[h, n + 1:] = hr["row_ptr"][-1] + base
        trp[h, :n + 1] = hr["t_row_ptr"] + base
        trp[h, n + 1:] = hr["t_row_ptr"][-1] + base
        cols.append(hr["col_idx"])
        tcols.append(hr["t_col_idx"])
        base += int(hr["row_ptr"][-1])
    ix = dict(perm=perm, bs=bs, nb=nb, rp=rp, ci=np.concatenate(cols).astype(np.int32), trp=trp,
              tci=np.concatenate(tcols).astype(np.int32))
    return c, ix


def _check(c, ix, n_idx=None):
    prob = B.make_problem(c.T, c.H, c.W, c.heads, c.head_dim)
    bad = (ctypes.c_int64 * 2)()
    st = B.prism_check_index(prob, ix["perm"], ix["bs"], ix["nb"], ix["rp"], ix["ci"], ix["trp"], ix["tci"],
                             ix["ci"].size if n_idx is None else n_idx, bad, check=False)
    return st, (bad[0], bad[1])


@pytest.mark.parametrize("name", ["tiny", "par_small", "par_heads"])
def test_oracle_index_passes(lib, name):
    c, ix = _index(name)
    assert _check(c, ix) == (B.PRISM_OK, (-1, -1))
    # the optional parts may be left out
    prob = B.make_problem(c.T, c.H, c.W, c.heads, c.head_dim)
    assert B.prism_check_index(prob, None, ix["bs"], ix["nb"], ix["rp"], ix["ci"], None, None, ix["ci"].size) == 0


def _copy(ix):
    return {k: v.copy() for k, v in ix.items()}


def test_malformed_indices_rejected(lib):
    c, ix = _index("par_small")           # two heads
    tiles = c.N // 64
    h1 = 1
    n1 = int(ix["nb"][h1])
    e0 = int(ix["rp"][h1, 0])            # first entry of head 1
    cases = []

    m = _copy(ix); m["ci"][e0] = n1                                    # key block out of range
    cases.append((m, (h1, 0)))
    m = _copy(ix); r = int(np.argmax(np.diff(ix["rp"][0]) >= 2)); a = int(ix["rp"][0, r])
    m["ci"][a], m["ci"][a + 1] = m["ci"][a + 1], m["ci"][a]           # a row out of order
    cases.append((m, (0, r)))
    m = _copy(ix); m["rp"][0, 1:] -= np.diff(ix["rp"][0])[0]; m["rp"][1] -= np.diff(ix["rp"][0])[0]
    m["ci"] = np.delete(m["ci"], np.arange(ix["rp"][0, 0], ix["rp"][0, 1]))
    m["tci"] = m["tci"]                                                # an empty row (transpose not updated)
    cases.append((m, (0, 0)))
    m = _copy(ix); m["rp"][h1] -= 1                                    # head 1 does not start where head 0 ends
    cases.append((m, (h1, 0)))
    m = _copy(ix); m["bs"][0, 1] = 3                                   # a block of three tiles
    cases.append((m, (0, 0)))
    m = _copy(ix); m["nb"][0] = tiles + 1                              # too many blocks
    cases.append((m, (0, -1)))
    m = _copy(ix); m["bs"][0, -1] = tiles - 1                          # tail entry changed
    cases.append((m, (0, tiles)))
    m = _copy(ix); m["perm"][h1, 5] = m["perm"][h1, 6]                 # perm not a bijection
    cases.append((m, (h1, 6)))
    m = _copy(ix); m["perm"][0, 0] = c.N                               # perm out of range
    cases.append((m, (0, 0)))
    m = _copy(ix); j = int(np.argmax(np.diff(ix["trp"][0]) >= 1)); m["tci"][ix["trp"][0, j]] += 10 ** 6
    cases.append((m, (0, tiles + 1 + j)))                              # transpose entry out of range
    for k, (m, where) in enumerate(cases):
        st, bad = _check(c, m)
        assert st == B.PRISM_EINDEX, (k, st)
        assert bad == where, (k, bad, where)
    # a capacity below the entries in use
    st, bad = _check(c, ix, n_idx=ix["ci"].size - 1)
    assert st == B.PRISM_EINDEX and bad[0] == 1


def test_transpose_must_match(lib):
    c, ix = _index("tiny")
    m = _copy(ix)
    # move one query block of a column to another column: both stay ascending
    tp = m["trp"][0]
    j = int(np.argmax(np.diff(tp) >= 1))
    i = int(m["tci"][tp[j]])
    m["tci"][tp[j]] = (i + 1) % int(ix["nb"][0])
    if np.diff(m["tci"][tp[j]:tp[j + 1]]).min(initial=1) > 0:
        st, bad = _check(c, m)
        assert st == B.PRISM_EINDEX and bad[0] == 0 and bad[1] >= c.N // 64 + 1


def test_argument_errors(lib):
    c, ix = _index("tiny")
    prob = B.make_problem(c.T, c.H, c.W, c.heads, c.head_dim)
    assert B.prism_check_index(prob, None, None, ix["nb"], ix["rp"], ix["ci"], None, None, 0, check=False) == \
        B.PRISM_EINVAL
    assert B.prism_check_index(prob, None, ix["bs"], ix["nb"], ix["rp"], ix["ci"], ix["trp"], None, 0,
                               check=False) == B.PRISM_EINVAL
    bad_grid = B.make_problem(12, c.H, c.W, c.heads, c.head_dim)
    assert B.prism_check_index(bad_grid, None, ix["bs"], ix["nb"], ix["rp"], ix["ci"], None, None, 0,
                               check=False) == B.PRISM_EGRID
