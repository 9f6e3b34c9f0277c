"""GPU checks of the forward-only inference path (prism_infer_fwd) through
the C ABI.  It runs the same kernels as the training path, head group by head
group in one reused workspace, so its output must equal the training path's
forward output (itself checked against the oracle in the parity tests) bit
for bit: in separate buffers, in place, with one head per pass, and at the
full forward-only and headline sizes.  A direct oracle check on a small
workload guards the chain."""

import math

import numpy as np
import pytest

import oracle as O
from workload import CONFIGS, generate

from parity_utils import (FWD_MAX_ABS, FWD_MEAN_ABS, LayerOnGpu, bf16_dev_to_f32, binding_params, fwd_errors, log,
                          oracle_params, to_dev)

pytestmark = pytest.mark.gpu


def _infer(wl, params, in_place=False):
    import torch
    from dynamic_block_sparse_macro_amd.pipeline import LayerShape, PrismInference
    c = wl.cfg
    inf = PrismInference(LayerShape(c.T, c.H, c.W, c.heads, c.head_dim), params)
    q, k, v = (to_dev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
    a = torch.from_numpy(wl.a).cuda()
    if in_place:
        inf.forward(q, k, v, a, q)
        o = q
    else:
        o = torch.full_like(q, float("nan"))
        inf.forward(q, k, v, a, o)
    torch.cuda.synchronize()
    return bf16_dev_to_f32(o), inf


CASES = [("tiny", {}), ("one_zone", {}), ("par_d64", {}), ("par_small", {}), ("par_small", dict(pass_heads=1)),
         ("par_cap", dict(pass_heads=1)), ("par_cap", dict(variant=O.VARIANT_TOPK_ONLY)),
         ("par_cap", dict(variant=O.VARIANT_TOPP_ONLY, pass_heads=1)),
         ("par_heads", dict(pass_heads=2))]   # five heads in passes of 2, 2 and 1


@pytest.mark.parametrize("name,over", CASES)
def test_infer_equals_training_forward(name, over):
    wl = generate(name)
    c = wl.cfg
    par = binding_params(c, **over)
    ref = LayerOnGpu(wl, params=par, backward=False).host()["o"]
    got, inf = _infer(wl, par)
    np.testing.assert_array_equal(got, ref)
    got2, _ = _infer(wl, par, in_place=True)
    np.testing.assert_array_equal(got2, ref)
    log(f"{name} {over}: inference output equals the training forward bit for bit (workspace "
        f"{inf.ws_bytes.value} bytes)")


def test_infer_against_oracle():
    """Direct check on the tiny workload: the oracle's whole forward layer."""
    wl = generate("tiny")
    c = wl.cfg
    got, _ = _infer(wl, binding_params(c))
    res = O.run_pipeline(wl.f32("q"), wl.f32("k"), wl.f32("v"), wl.a, c.T, c.H, c.W, oracle_params(c))
    if any(hr["sel"]["ties"] for hr in res["heads"]):
        pytest.skip("tied selection rows: covered by the training-path parity test")
    for h, hr in enumerate(res["heads"]):
        mx, mean = fwd_errors(got[h], hr["o"])
        log(f"head {h}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= FWD_MAX_ABS and mean <= FWD_MEAN_ABS


@pytest.mark.slow
@pytest.mark.parametrize("name", ["720p", "2k"])
def test_infer_fullsize(name):
    """The forward-only 720p clip (one pass of four heads) and the 2K clip
    (two passes of one head) against the training forward, bit for bit, and
    the inference workspace against the training path's device bytes."""
    from dynamic_block_sparse_macro_amd.pipeline import training_path_bytes
    wl = generate(CONFIGS[name])
    c = wl.cfg
    par = binding_params(c)
    run = LayerOnGpu(wl, params=par, backward=False)
    ref = run.host()["o"]
    got, inf = _infer(wl, par)
    np.testing.assert_array_equal(got, ref)
    tr = training_path_bytes(run.layer, int(sum(run.layer.nnz)))
    log(f"{name}: inference workspace {inf.ws_bytes.value / 2**20:.1f} MiB vs training path "
        f"{tr['total'] / 2**20:.1f} MiB ({100 * (1 - inf.ws_bytes.value / tr['total']):.1f}% less)")
    assert inf.ws_bytes.value < tr["total"]
