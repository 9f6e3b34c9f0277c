"""Write tiny_snapshot.json: the oracle's discrete decisions and a few output
values on the seeded tiny workload (8x16x16 grid, one head, head_dim 64).

Calls only the oracle and the seeded generator.  Run from the repository
root:  python tests/golden/make_tiny_snapshot.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from workload import generate  # noqa: E402


def snapshot() -> dict:
    w = generate("tiny")
    c = w.cfg
    P = O.Params(top_k=c.top_k, top_p=c.top_p, density_cap=c.density_cap)
    r = O.run_pipeline(w.f32("q"), w.f32("k"), w.f32("v"), w.a, c.T, c.H, c.W, P, do=w.f32("do"))
    h = r["heads"][0]
    probe = [0, 517, 1023, 2047]
    return dict(
        workload="tiny", params=dict(top_k=c.top_k, top_p=c.top_p, eps=P.eps, tau128=P.tau128, tau256=P.tau256),
        g=r["zone"]["g"][0].tolist(), rho=r["zone"]["rho"][0].tolist(),
        shape_id=r["plan"]["shape_id"][0].tolist(), blk_start=h["blk_start"].tolist(),
        row_ptr=h["row_ptr"].tolist(), col_idx=h["col_idx"].tolist(),
        o_probe={str(t): h["o"][t, :4].tolist() for t in probe},
        dq_probe={str(t): h["dq"][t, :4].tolist() for t in probe},
    )


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_snapshot.json")
    with open(out, "w") as f:
        json.dump(snapshot(), f, indent=1)
    print("wrote", out)
