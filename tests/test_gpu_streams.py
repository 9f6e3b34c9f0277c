"""GPU checks of the stream contract of the C ABI: every entry point enqueues
its work on the stream it is given, so the whole layer (training forward and
backward, and the forward-only path) run on side streams, two layers at a
time, gives results bitwise equal to the same calls on the default stream."""

import numpy as np
import pytest

from workload import generate

from parity_utils import LayerOnGpu, bf16_dev_to_f32, binding_params, log, to_dev

pytestmark = pytest.mark.gpu


def _enqueue_layer(wl, stream):
    """Upload the inputs and run forward + backward + the forward-only path
    on `stream` without synchronising (apart from the selection's own
    read-back); returns the objects holding the results."""
    import torch
    from dynamic_block_sparse_macro_amd.pipeline import LayerShape, PrismInference, PrismLayer
    c = wl.cfg
    shape = LayerShape(c.T, c.H, c.W, c.heads, c.head_dim)
    with torch.cuda.stream(stream):
        q, k, v, do = (to_dev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits, wl.do_bits))
        a = torch.from_numpy(wl.a).cuda()
        layer = PrismLayer(shape, binding_params(c))
        o = torch.empty_like(q)
        layer.forward(q, k, v, a, o)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        layer.attn_bwd(o, do, dq, dk, dv)
        inf = PrismInference(shape, binding_params(c))
        o_inf = torch.empty_like(q)
        inf.forward(q, k, v, a, o_inf)
    return dict(layer=layer, o=o, dq=dq, dk=dk, dv=dv, o_inf=o_inf, keep=(q, k, v, do, a, inf))


def test_side_streams_match_default_stream():
    import torch
    wl = generate("par_small")
    ref = LayerOnGpu(wl, backward=True).host()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    runs = [_enqueue_layer(wl, s) for s in (s1, s2)]
    torch.cuda.synchronize()
    for i, r in enumerate(runs):
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_array_equal(bf16_dev_to_f32(r[key]), ref[key], err_msg=f"stream {i}: {key}")
        np.testing.assert_array_equal(bf16_dev_to_f32(r["o_inf"]), ref["o"], err_msg=f"stream {i}: inference")
        np.testing.assert_array_equal(r["layer"].lse.cpu().numpy(), ref["lse"])
        for ia, ib in zip(r["layer"].index_host(), ref["index"]):
            for key in ("perm", "blk_start", "row_ptr", "col_idx", "t_row_ptr", "t_col_idx"):
                np.testing.assert_array_equal(ia[key], ib[key], err_msg=key)
    log("two layers on two side streams: bitwise equal to the default stream")
