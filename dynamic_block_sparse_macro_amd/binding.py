"""ctypes binding of libprism.so: argument marshalling only.

Every function here has the name and argument order of the C entry point it
wraps (see include/prism.h); tensors are passed as torch tensors (their device
pointers are used) or None for NULL, streams as torch streams or None.  The
compute happens in the HIP library; there is no fallback: if the library is
missing, loading fails with an error.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libprism.so")

PRISM_OK = 0
PRISM_EINVAL = -1
PRISM_EGRID = -2
PRISM_EDIM = -3
PRISM_EPARAM = -4
PRISM_ECAPACITY = -5
PRISM_EWORKSPACE = -6
PRISM_EHIP = -7
PRISM_EINDEX = -8

VARIANT_FIXED_SHAPE = 1
VARIANT_TOPK_ONLY = 2
VARIANT_TOPP_ONLY = 4
VARIANT_VISUAL_ONLY = 8
VARIANT_AUDIO_ONLY = 16
VARIANT_RHO_MAX_AUDIO = 32

ENTRY_POINTS = ("prism_zone_stats", "prism_plan_shapes", "prism_select_blocks", "prism_attn_fwd",
                "prism_attn_bwd", "prism_dense_attn_fwd", "prism_dense_attn_bwd", "prism_a2v_norms", "prism_infer_fwd",
                "prism_check_index", "prism_attn_fwd_noalloc", "prism_sclk_probe", "prism_strerror")


class PrismError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("head_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64)]


class Params(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_double), ("tau128", ctypes.c_double), ("tau256", ctypes.c_double),
                ("top_k", ctypes.c_int32), ("variant", ctypes.c_int32), ("top_p", ctypes.c_double),
                ("density_cap", ctypes.c_double), ("scale", ctypes.c_double),
                ("fixed_shape", ctypes.c_int32), ("pass_heads", ctypes.c_int32)]


def make_problem(T, H, W, heads, head_dim, head_stride=None, token_stride=None) -> Problem:
    ts = head_dim if token_stride is None else token_stride
    hs = T * H * W * ts if head_stride is None else head_stride
    return Problem(T, H, W, heads, head_dim, hs, ts)


def make_params(top_k=16, top_p=0.9, density_cap=1.0, eps=1e-6, tau128=0.5, tau256=0.25, scale=0.0,
                variant=0, fixed_shape=0, pass_heads=0) -> Params:
    return Params(eps, tau128, tau256, top_k, variant, top_p, density_cap, scale, fixed_shape, pass_heads)


_lib = None
_vp = ctypes.c_void_p
_P = ctypes.POINTER


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libprism.so (built by dynamic_block_sparse_macro_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m dynamic_block_sparse_macro_amd.build`")
    lib = ctypes.CDLL(path)
    pp, pr = _P(Problem), _P(Params)
    sig = {
        "prism_zone_stats": [pp, pr, _vp, _vp, _vp, _vp, _vp, _vp],
        "prism_plan_shapes": [pp, pr, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        "prism_select_blocks": [pp, pr, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                _vp, _vp, _vp, _vp, _P(ctypes.c_size_t), _vp],
        "prism_attn_fwd": [pp, pr] + [_vp] * 12 + [_P(ctypes.c_size_t), _vp],
        "prism_attn_bwd": [pp, pr] + [_vp] * 18 + [_P(ctypes.c_size_t), _vp],
        "prism_dense_attn_fwd": [pp, pr, _vp, _vp, _vp, _vp, _vp, _vp, _P(ctypes.c_size_t), _vp],
        "prism_dense_attn_bwd": [pp, pr] + [_vp] * 10 + [_P(ctypes.c_size_t), _vp],
        "prism_a2v_norms": [_vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, _vp, _vp],
        "prism_infer_fwd": [pp, pr, _vp, _vp, _vp, _vp, _vp, _vp, _P(ctypes.c_size_t), _vp],
        "prism_check_index": [pp] + [_vp] * 7 + [ctypes.c_int64, _vp],
        "prism_attn_fwd_noalloc": [pp, pr] + [_vp] * 12,
        "prism_sclk_probe": [_P(ctypes.c_double), _vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.prism_strerror.argtypes = [ctypes.c_int]
    lib.prism_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().prism_strerror(status).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Array):
        return ctypes.addressof(x)
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _stream(s):
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(name: str, status: int, allow=()) -> int:
    if status != PRISM_OK and status not in allow:
        raise PrismError(name, status, strerror(status))
    return status


def prism_zone_stats(prob, par, v, a, zstats, g, rho, stream=None, check=True):
    st = load_library().prism_zone_stats(ctypes.byref(prob), ctypes.byref(par), _ptr(v), _ptr(a), _ptr(zstats),
                                         _ptr(g), _ptr(rho), _stream(stream))
    return _check("prism_zone_stats", st) if check else st


def prism_plan_shapes(prob, par, g, rho, shape_id, perm, blk_start, n_blocks, stream=None, check=True):
    st = load_library().prism_plan_shapes(ctypes.byref(prob), ctypes.byref(par), _ptr(g), _ptr(rho), _ptr(shape_id),
                                          _ptr(perm), _ptr(blk_start), _ptr(n_blocks), _stream(stream))
    return _check("prism_plan_shapes", st) if check else st


def prism_select_blocks(prob, par, q, k, v, perm, blk_start, n_blocks, qp, kp, vp, row_ptr, col_idx, col_cap,
                        t_row_ptr, t_col_idx, nnz_host, ws, ws_bytes, stream=None, check=True):
    """nnz_host: ctypes int64 array of `heads` entries; ws_bytes: ctypes.c_size_t."""
    st = load_library().prism_select_blocks(
        ctypes.byref(prob), ctypes.byref(par), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(blk_start),
        _ptr(n_blocks), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(row_ptr), _ptr(col_idx), int(col_cap),
        _ptr(t_row_ptr), _ptr(t_col_idx), _ptr(nnz_host), _ptr(ws), _ref(ws_bytes), _stream(stream))
    return _check("prism_select_blocks", st, allow=(PRISM_ECAPACITY,)) if check else st


def prism_attn_fwd(prob, par, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, o_lo, lse, ws, ws_bytes,
                   stream=None, check=True):
    st = load_library().prism_attn_fwd(ctypes.byref(prob), ctypes.byref(par), _ptr(qp), _ptr(kp), _ptr(vp),
                                       _ptr(perm), _ptr(blk_start), _ptr(n_blocks), _ptr(row_ptr), _ptr(col_idx),
                                       _ptr(o), _ptr(o_lo), _ptr(lse), _ptr(ws), _ref(ws_bytes), _stream(stream))
    return _check("prism_attn_fwd", st) if check else st


def prism_attn_fwd_noalloc(prob, par, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, o_lo, lse,
                           stream=None, check=True):
    st = load_library().prism_attn_fwd_noalloc(ctypes.byref(prob), ctypes.byref(par), _ptr(qp), _ptr(kp), _ptr(vp),
                                               _ptr(perm), _ptr(blk_start), _ptr(n_blocks), _ptr(row_ptr),
                                               _ptr(col_idx), _ptr(o), _ptr(o_lo), _ptr(lse), _stream(stream))
    return _check("prism_attn_fwd_noalloc", st) if check else st


def prism_attn_bwd(prob, par, qp, kp, vp, o, o_lo, dout, lse, perm, blk_start, n_blocks, row_ptr, col_idx,
                   t_row_ptr, t_col_idx, dq, dk, dv, ws, ws_bytes, stream=None, check=True):
    st = load_library().prism_attn_bwd(
        ctypes.byref(prob), ctypes.byref(par), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(o), _ptr(o_lo), _ptr(dout),
        _ptr(lse),
        _ptr(perm), _ptr(blk_start), _ptr(n_blocks), _ptr(row_ptr), _ptr(col_idx), _ptr(t_row_ptr),
        _ptr(t_col_idx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _ref(ws_bytes), _stream(stream))
    return _check("prism_attn_bwd", st) if check else st


def prism_dense_attn_fwd(prob, par, q, k, v, o, lse, ws, ws_bytes, stream=None, check=True):
    st = load_library().prism_dense_attn_fwd(ctypes.byref(prob), ctypes.byref(par), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(o), _ptr(lse), _ptr(ws), _ref(ws_bytes), _stream(stream))
    return _check("prism_dense_attn_fwd", st) if check else st


def prism_dense_attn_bwd(prob, par, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, stream=None, check=True):
    st = load_library().prism_dense_attn_bwd(ctypes.byref(prob), ctypes.byref(par), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                             _ref(ws_bytes), _stream(stream))
    return _check("prism_dense_attn_bwd", st) if check else st


def prism_a2v_norms(h_hat, n_tokens, channels, token_stride, a, stream=None, check=True):
    st = load_library().prism_a2v_norms(_ptr(h_hat), int(n_tokens), int(channels), int(token_stride), _ptr(a),
                                        _stream(stream))
    return _check("prism_a2v_norms", st) if check else st


def prism_infer_fwd(prob, par, q, k, v, a, o, ws, ws_bytes, stream=None, check=True):
    st = load_library().prism_infer_fwd(ctypes.byref(prob), ctypes.byref(par), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                        _ptr(o), _ptr(ws), _ref(ws_bytes), _stream(stream))
    return _check("prism_infer_fwd", st) if check else st


def prism_sclk_probe(stream=None) -> float:
    """Shader clock (GHz) under a sustained MFMA load; synchronises the stream."""
    ghz = ctypes.c_double(0.0)
    _check("prism_sclk_probe", load_library().prism_sclk_probe(ctypes.byref(ghz), _stream(stream)))
    return ghz.value


def prism_check_index(prob, perm, blk_start, n_blocks, row_ptr, col_idx, t_row_ptr, t_col_idx, n_idx, bad=None,
                      check=True):
    """Host arrays (numpy int32, C-contiguous, or None); bad: ctypes int64
    array of 2 (optional).  Returns the status (raises unless check=False)."""
    def host(a):
        if a is None:
            return None
        assert a.dtype.str == "<i4" and a.flags["C_CONTIGUOUS"], "int32 C-contiguous host array expected"
        return a.ctypes.data
    st = load_library().prism_check_index(ctypes.byref(prob), host(perm), host(blk_start), host(n_blocks),
                                          host(row_ptr), host(col_idx), host(t_row_ptr), host(t_col_idx),
                                          int(n_idx), _ptr(bad))
    return _check("prism_check_index", st) if check else st
