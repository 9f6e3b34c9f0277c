"""GPU checks of the C ABI's layout and capacity contracts.

* Strided THW tensors (heads interleaved inside each token, and the fused
  [token][q|k|v][head][channel] layout of a QKV projection) give results
  bitwise equal to the contiguous [head][token][channel] layout, through the
  training path (forward and backward) and the forward-only path (in place).
* A block index larger than col_cap is reported with PRISM_ECAPACITY, the
  per-head counts in nnz_host, and no index entry written; a retry with the
  reported capacity gives the same index as a single large call.
"""

import ctypes

import numpy as np
import pytest

from workload import generate

from parity_utils import LayerOnGpu, bf16_dev_to_f32, binding_params, log, to_dev

pytestmark = pytest.mark.gpu


def _run_strided(wl, fused: bool):
    """Run the layer on strided copies of the workload; returns host arrays
    in [head][token][channel] order."""
    import torch
    from dynamic_block_sparse_macro_amd.pipeline import LayerShape, PrismLayer
    c = wl.cfg
    H, N, D = c.heads, c.N, c.head_dim

    def interleave(bits):                       # [H][N][D] -> [N][H][D]
        return np.ascontiguousarray(np.transpose(bits, (1, 0, 2)))

    if fused:
        # [N][3][H][D]: q, k, v of a token side by side; o, dO, dq, dk, dv in
        # buffers of the same shape (slot 0)
        qkv = np.stack([interleave(wl.q_bits), interleave(wl.k_bits), interleave(wl.v_bits)], axis=1)
        dev = to_dev(qkv)
        q, k, v = dev[:, 0], dev[:, 1], dev[:, 2]
        token_stride, head_stride = 3 * H * D, D

        def like():
            return torch.full((N, 3, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")[:, 0]
        do = like()
        do.copy_(to_dev(interleave(wl.do_bits)))
    else:
        q, k, v, do = (to_dev(interleave(b)) for b in (wl.q_bits, wl.k_bits, wl.v_bits, wl.do_bits))
        token_stride, head_stride = H * D, D

        def like():
            return torch.full((N, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    a = torch.from_numpy(wl.a).cuda()
    layer = PrismLayer(LayerShape(c.T, c.H, c.W, H, D), binding_params(c), head_stride=head_stride,
                       token_stride=token_stride)
    o, dq, dk, dv = like(), like(), like(), like()
    layer.forward(q, k, v, a, o)
    layer.attn_bwd(o, do, dq, dk, dv)
    torch.cuda.synchronize()

    def host(t):                               # strided [N][H][D] view -> [H][N][D]
        return np.transpose(bf16_dev_to_f32(t.contiguous()), (1, 0, 2))
    out = dict(o=host(o), dq=host(dq), dk=host(dk), dv=host(dv), lse=layer.lse.cpu().numpy(),
               index=layer.index_host())

    # forward-only path, in place over q
    from dynamic_block_sparse_macro_amd.pipeline import PrismInference
    inf = PrismInference(layer.shape, binding_params(c), head_stride=head_stride, token_stride=token_stride)
    qc = q.clone() if not fused else None
    if fused:
        buf = to_dev(qkv)
        qc, kc, vc = buf[:, 0], buf[:, 1], buf[:, 2]
    else:
        kc, vc = k, v
    inf.forward(qc, kc, vc, a, qc)
    torch.cuda.synchronize()
    out["o_infer"] = host(qc)
    return out


@pytest.mark.parametrize("name,fused", [("par_small", False), ("par_small", True), ("par_d64", True)])
def test_strided_layouts(name, fused):
    wl = generate(name)
    ref = LayerOnGpu(wl, backward=True).host()
    got = _run_strided(wl, fused)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["lse"], ref["lse"])
    np.testing.assert_array_equal(got["o_infer"], ref["o"])
    for ia, ib in zip(got["index"], ref["index"]):
        for key in ("perm", "blk_start", "row_ptr", "col_idx", "t_row_ptr", "t_col_idx"):
            np.testing.assert_array_equal(ia[key], ib[key], err_msg=key)
    log(f"{name} ({'fused qkv' if fused else 'heads interleaved'}): bitwise equal to the contiguous layout")


def test_capacity_error_writes_no_index():
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    wl = generate("par_cap")
    c = wl.cfg
    full = LayerOnGpu(wl, backward=False)
    L = full.layer
    want = [int(x) for x in L.nnz]
    # a second select call with room for fewer pairs than selected
    rp = torch.full_like(L.row_ptr, -7)
    trp = torch.full_like(L.t_row_ptr, -7)
    cap = sum(want) - 1
    col = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    tcol = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    nnz = (ctypes.c_int64 * c.heads)()
    st = B.prism_select_blocks(L.prob, L.params, full.q, full.k, full.v, L.perm, L.blk_start, L.n_blocks, L.qp, L.kp,
                               L.vp, rp, col, cap, trp, tcol, nnz, L.sel_ws, L.sel_ws_bytes, check=False)
    torch.cuda.synchronize()
    assert st == B.PRISM_ECAPACITY
    assert list(nnz) == want
    for t in (rp, trp, col, tcol):
        assert bool((t == -7).all()), "an index buffer was written despite the capacity error"
    # retry with exactly the reported capacity: same index as the first call
    cap = sum(nnz)
    col = torch.empty(cap, dtype=torch.int32, device="cuda")
    tcol = torch.empty_like(col)
    st = B.prism_select_blocks(L.prob, L.params, full.q, full.k, full.v, L.perm, L.blk_start, L.n_blocks, L.qp, L.kp,
                               L.vp, rp, col, cap, trp, tcol, nnz, L.sel_ws, L.sel_ws_bytes, check=False)
    torch.cuda.synchronize()
    assert st == B.PRISM_OK
    np.testing.assert_array_equal(rp.cpu().numpy(), L.row_ptr.cpu().numpy())
    np.testing.assert_array_equal(trp.cpu().numpy(), L.t_row_ptr.cpu().numpy())
    np.testing.assert_array_equal(col.cpu().numpy(), L.col_idx[:cap].cpu().numpy())
    np.testing.assert_array_equal(tcol.cpu().numpy(), L.t_col_idx[:cap].cpu().numpy())
    log(f"capacity error reported with counts {want}; retry equals the single call")


def test_layer_capacity_retry():
    """PrismLayer grows its index on PRISM_ECAPACITY and retries: results equal
    those of a layer that had room from the start."""
    wl = generate("par_small")
    a = LayerOnGpu(wl, backward=True).host()
    b = LayerOnGpu(wl, backward=True, layer_kw=dict(col_cap=1)).host()
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
