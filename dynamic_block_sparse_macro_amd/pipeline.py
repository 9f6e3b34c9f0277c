"""Device buffers for one Prism attention layer, and the calls that run it.

PrismLayer owns the intermediate buffers of the five C entry points (as
torch tensors, i.e. device memory from torch's allocator) and calls them in
order on the current torch stream.  Every step runs in libprism.so.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class LayerShape:
    T: int
    H: int
    W: int
    heads: int
    head_dim: int

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Z(self) -> int:
        return self.N // 512

    @property
    def tiles(self) -> int:
        return self.N // 64


def a2v_norms(h_hat: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """a[n] = |h_hat[n]|_2 (float32) for a bf16 [N][C] tensor whose rows are
    THW tokens: the audio guidance map the next layer's zone statistics
    read.  Runs prism_a2v_norms on the current stream."""
    if h_hat.dtype != torch.bfloat16 or h_hat.dim() != 2 or h_hat.stride(1) != 1:
        raise ValueError("h_hat must be a bf16 [N][C] tensor with unit channel stride")
    n, c = h_hat.shape
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=h_hat.device)
    B.prism_a2v_norms(h_hat, n, c, h_hat.stride(0), out, stream=torch.cuda.current_stream())
    return out


class PrismLayer:
    def __init__(self, shape: LayerShape, params: B.Params, device="cuda", col_cap: int | None = None,
                 head_stride: int | None = None, token_stride: int | None = None):
        self.shape = s = shape
        self.params = params
        self.device = device
        self.prob = B.make_problem(s.T, s.H, s.W, s.heads, s.head_dim, head_stride, token_stride)
        dev = dict(device=device)
        h, Z, N, D, t = s.heads, s.Z, s.N, s.head_dim, s.tiles
        self.zstats = torch.empty(h, Z, 8, dtype=torch.float64, **dev)
        self.g = torch.empty(h, Z, 3, dtype=torch.float64, **dev)
        self.rho = torch.empty(h, Z, dtype=torch.float64, **dev)
        self.shape_id = torch.empty(h, Z, dtype=torch.uint8, **dev)
        self.perm = torch.empty(h, N, dtype=torch.int32, **dev)
        self.blk_start = torch.empty(h, t + 1, dtype=torch.int32, **dev)
        self.n_blocks = torch.empty(h, dtype=torch.int32, **dev)
        self.qp = torch.empty(h, N, D, dtype=torch.bfloat16, **dev)
        self.kp = torch.empty_like(self.qp)
        self.vp = torch.empty_like(self.qp)
        self.row_ptr = torch.empty(h, t + 1, dtype=torch.int32, **dev)
        self.t_row_ptr = torch.empty_like(self.row_ptr)
        self.col_cap = col_cap if col_cap is not None else max(1, h * t * min(t, 512))
        self.col_idx = torch.empty(self.col_cap, dtype=torch.int32, **dev)
        self.t_col_idx = torch.empty_like(self.col_idx)
        self.lse = torch.empty(h, N, dtype=torch.float32, **dev)
        # low bf16 parts of the forward output (block order), for the backward's rowsum(dO * O)
        self.o_lo = torch.empty(h, N, D, dtype=torch.bfloat16, **dev)
        self.nnz = (ctypes.c_int64 * h)()
        self.sel_ws_bytes = ctypes.c_size_t(0)
        B.prism_select_blocks(self.prob, params, None, None, None, None, None, None, None, None, None, None, None,
                              0, None, None, None, None, self.sel_ws_bytes)
        self.sel_ws = torch.empty(self.sel_ws_bytes.value, dtype=torch.uint8, **dev)
        self.fwd_ws_bytes = ctypes.c_size_t(0)
        B.prism_attn_fwd(self.prob, params, *([None] * 12), self.fwd_ws_bytes)
        self.fwd_ws = torch.empty(self.fwd_ws_bytes.value, dtype=torch.uint8, **dev)
        self.bwd_ws_bytes = ctypes.c_size_t(0)
        B.prism_attn_bwd(self.prob, params, *([None] * 18), self.bwd_ws_bytes)
        self.bwd_ws = None

    def stream(self):
        return torch.cuda.current_stream(self.device)

    # -- steps ---------------------------------------------------------------
    def zone_stats(self, v, a):
        B.prism_zone_stats(self.prob, self.params, v, a, self.zstats, self.g, self.rho, self.stream())

    def plan_shapes(self):
        B.prism_plan_shapes(self.prob, self.params, self.g, self.rho, self.shape_id, self.perm, self.blk_start,
                            self.n_blocks, self.stream())

    def select_blocks(self, q, k, v):
        st = B.prism_select_blocks(self.prob, self.params, q, k, v, self.perm, self.blk_start, self.n_blocks,
                                   self.qp, self.kp, self.vp, self.row_ptr, self.col_idx, self.col_cap,
                                   self.t_row_ptr, self.t_col_idx, self.nnz, self.sel_ws, self.sel_ws_bytes,
                                   self.stream())
        if st == B.PRISM_ECAPACITY:
            self.col_cap = int(sum(self.nnz))
            self.col_idx = torch.empty(self.col_cap, dtype=torch.int32, device=self.device)
            self.t_col_idx = torch.empty_like(self.col_idx)
            B.prism_select_blocks(self.prob, self.params, q, k, v, self.perm, self.blk_start, self.n_blocks,
                                  self.qp, self.kp, self.vp, self.row_ptr, self.col_idx, self.col_cap,
                                  self.t_row_ptr, self.t_col_idx, self.nnz, self.sel_ws, self.sel_ws_bytes,
                                  self.stream())
        return [int(x) for x in self.nnz]

    def attn_fwd(self, o):
        B.prism_attn_fwd(self.prob, self.params, self.qp, self.kp, self.vp, self.perm, self.blk_start,
                         self.n_blocks, self.row_ptr, self.col_idx, o, self.o_lo, self.lse, self.fwd_ws,
                         self.fwd_ws_bytes, self.stream())

    def attn_bwd(self, o, do, dq, dk, dv):
        if self.bwd_ws is None:
            self.bwd_ws = torch.empty(self.bwd_ws_bytes.value, dtype=torch.uint8, device=self.device)
        B.prism_attn_bwd(self.prob, self.params, self.qp, self.kp, self.vp, o, self.o_lo, do, self.lse, self.perm,
                         self.blk_start, self.n_blocks, self.row_ptr, self.col_idx, self.t_row_ptr, self.t_col_idx,
                         dq, dk, dv, self.bwd_ws, self.bwd_ws_bytes, self.stream())

    def forward(self, q, k, v, a, o):
        self.zone_stats(v, a)
        self.plan_shapes()
        nnz = self.select_blocks(q, k, v)
        self.attn_fwd(o)
        return nnz

    # -- host copies of the block index ---------------------------------------
    def index_host(self):
        """Per head: (perm, blk_start, row_ptr, col_idx, t_row_ptr, t_col_idx) as numpy, local offsets."""
        out = []
        nb = self.n_blocks.cpu().numpy()
        rp_all = self.row_ptr.cpu().numpy()
        trp_all = self.t_row_ptr.cpu().numpy()
        col = self.col_idx.cpu().numpy()
        tcol = self.t_col_idx.cpu().numpy()
        perm = self.perm.cpu().numpy()
        bs_all = self.blk_start.cpu().numpy()
        for h in range(self.shape.heads):
            n = int(nb[h])
            rp = rp_all[h, :n + 1].astype("int64")
            trp = trp_all[h, :n + 1].astype("int64")
            out.append(dict(n_blocks=n, perm=perm[h], blk_start=bs_all[h, :n + 1].astype("int64"),
                            row_ptr=rp - rp[0], col_idx=col[rp[0]:rp[-1]].astype("int64"),
                            t_row_ptr=trp - trp[0], t_col_idx=tcol[trp[0]:trp[-1]].astype("int64")))
        return out


class PrismInference:
    """The forward-only layer (prism_infer_fwd): one call, one workspace, no
    LSE and no key-major index kept.  forward(q, k, v, a, o) may run in
    place (o is q)."""

    def __init__(self, shape: LayerShape, params: B.Params, device="cuda", head_stride: int | None = None,
                 token_stride: int | None = None):
        s = shape
        self.shape = s
        self.params = params
        self.device = device
        self.prob = B.make_problem(s.T, s.H, s.W, s.heads, s.head_dim, head_stride, token_stride)
        self.ws_bytes = ctypes.c_size_t(0)
        B.prism_infer_fwd(self.prob, params, None, None, None, None, None, None, self.ws_bytes)
        self.ws = torch.empty(self.ws_bytes.value, dtype=torch.uint8, device=device)

    def forward(self, q, k, v, a, o):
        B.prism_infer_fwd(self.prob, self.params, q, k, v, a, o, self.ws, self.ws_bytes,
                          torch.cuda.current_stream(self.device))


def training_path_bytes(layer: "PrismLayer", nnz_total: int) -> dict:
    """Device bytes of the training path per layer beyond the caller's
    tensors: what the forward keeps for the backward (permuted operands, the
    low parts of O, LSE, permutation, block starts, both block indices sized
    to the selected pairs) and the larger of the two transient workspaces
    (selection, backward), which a caller can share."""
    s = layer.shape
    h, N, D, t, Z = s.heads, s.N, s.head_dim, s.tiles, s.Z
    kept = (4 * h * N * D * 2 + h * N * 4 + h * N * 4 + h * (t + 1) * 4 + h * 4 + 2 * h * (t + 1) * 4
            + 2 * nnz_total * 4 + h * Z * (8 + 3 + 1) * 8 + h * Z)
    transient = max(layer.sel_ws_bytes.value, layer.bwd_ws_bytes.value, layer.fwd_ws_bytes.value)
    return dict(kept=kept, transient=transient, total=kept + transient)


class DenseAttention:
    """Full attention on the same kernels (every key tile selected)."""

    def __init__(self, shape: LayerShape, params: B.Params, device="cuda"):
        s = shape
        self.prob = B.make_problem(s.T, s.H, s.W, s.heads, s.head_dim)
        self.params = params
        self.device = device
        self.lse = torch.empty(s.heads, s.N, dtype=torch.float32, device=device)
        self.fwd_bytes = ctypes.c_size_t(0)
        B.prism_dense_attn_fwd(self.prob, params, None, None, None, None, None, None, self.fwd_bytes)
        self.bwd_bytes = ctypes.c_size_t(0)
        B.prism_dense_attn_bwd(self.prob, params, *([None] * 9), None, self.bwd_bytes)
        self.ws = torch.empty(max(self.fwd_bytes.value, self.bwd_bytes.value), dtype=torch.uint8, device=device)
        self.ws_bytes = ctypes.c_size_t(self.ws.numel())

    def forward(self, q, k, v, o):
        B.prism_dense_attn_fwd(self.prob, self.params, q, k, v, o, self.lse, self.ws, self.ws_bytes,
                               torch.cuda.current_stream(self.device))

    def backward(self, q, k, v, o, do, dq, dk, dv):
        B.prism_dense_attn_bwd(self.prob, self.params, q, k, v, o, do, self.lse, dq, dk, dv, self.ws, self.ws_bytes,
                               torch.cuda.current_stream(self.device))
