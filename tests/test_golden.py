"""The oracle against the stored fixtures under tests/golden/."""
import json
import math
import os

import numpy as np

import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_closed_form_fixture():
    cf = json.load(open(os.path.join(HERE, "closed_forms.json")))
    assert O.ZONE == cf["zone_edge"]["value"]
    assert sorted(set(O.CANDIDATE_VOLUMES.tolist())) == cf["volumes"]["value"]
    assert len(O.CANDIDATES) == cf["n_candidates"]["value"]
    for vol, shapes in cf["candidates_by_volume"]["value"].items():
        assert O.CANDIDATES[O.CANDIDATE_VOLUMES == int(vol)].tolist() == shapes
    p = O.Params()
    assert (p.tau128, p.tau256) == (cf["thresholds"]["tau128"], cf["thresholds"]["tau256"])
    e = cf["ell_star_exact"]
    np.testing.assert_allclose(O.ell_star(np.array(e["g"]), e["B"]), e["ell"], atol=1e-14)
    iso = cf["ell_star_isotropic"]
    np.testing.assert_allclose(O.ell_star(np.full(3, 0.2), iso["B"]), iso["ell"], atol=1e-14)
    _, _, idx, dist = O.quantise_shape(O.ell_star(np.full(3, 0.2), iso["B"]), iso["B"])
    best = [O.CANDIDATES[i].tolist() for i, d in zip(idx, dist) if d <= dist.min() + 1e-12]
    assert sorted(best) == sorted(iso["tie"])
    assert math.isclose(dist.min(), 2.0 / 3.0, abs_tol=1e-14)


def test_tiny_snapshot_regression():
    import sys
    sys.path.insert(0, HERE)
    from make_tiny_snapshot import snapshot
    want = json.load(open(os.path.join(HERE, "tiny_snapshot.json")))
    got = snapshot()
    for key in ("shape_id", "blk_start", "row_ptr", "col_idx"):
        assert got[key] == want[key], key
    np.testing.assert_allclose(got["g"], want["g"], rtol=1e-14)
    np.testing.assert_allclose(got["rho"], want["rho"], rtol=1e-14)
    for t in want["o_probe"]:
        np.testing.assert_allclose(got["o_probe"][t], want["o_probe"][t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got["dq_probe"][t], want["dq_probe"][t], rtol=1e-12, atol=1e-14)
