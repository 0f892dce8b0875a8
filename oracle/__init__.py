"""CPU oracle for MoE expert-parallel dispatch and combine (ctypes over moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the package smoke check and the
CPU-baseline leg of bench.py may import this module.  It shares no code with
the HIP product path and never imports it.

What each function computes is stated in moe_oracle.c, with the page and
section it follows (the CANN "low_latency_dispatch" page: Function / Formula,
Constraints, Deterministic Computation, Example; the DeepEP issue "#84
Questions on Profiling dispatch_t ..." for -1 slots and expert ownership).
All arrays are numpy, host memory, C-contiguous.  bf16 tensors are carried as
uint16 bit patterns.
"""
import ctypes
import os
from collections import namedtuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_oracle.so")

Shape = namedtuple(
    "Shape",
    "num_tokens hidden topk num_experts num_ranks zero_expert_num copy_expert_num "
    "const_expert_num num_max_dispatch_tokens_per_rank",
)


class _CShape(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in Shape._fields]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.orc_check_shape.argtypes = [P]
        L.orc_check_shape.restype = ctypes.c_int
        L.orc_layout.argtypes = [P] * 12
        L.orc_layout.restype = ctypes.c_int
        L.orc_layout_ex.argtypes = [P, ctypes.c_int64] + [P] * 11
        L.orc_layout_ex.restype = ctypes.c_int
        L.orc_rank_capacity.argtypes = [P]
        L.orc_rank_capacity.restype = ctypes.c_int64
        L.orc_quant_token.argtypes = [ctypes.c_int, P, P, P, P]
        L.orc_quant_token.restype = None
        L.orc_quant_static.argtypes = [ctypes.c_int, P, P, P]
        L.orc_quant_static.restype = None
        L.orc_dispatch.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P, P, P, P, P]
        L.orc_dispatch.restype = ctypes.c_int
        L.orc_combine.argtypes = [P] * 11
        L.orc_combine.restype = ctypes.c_int
        L.orc_double_to_bf16.argtypes = [ctypes.c_double]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def make_shape(T, H, K, E, P, Z=0, C=0, Kc=0, num_max=0):
    return Shape(T, H, K, E, P, Z, C, Kc, num_max)


def _cs(shape):
    return _CShape(*[int(v) for v in shape])


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _arr(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def check_shape(shape):
    cs = _cs(shape)
    return lib().orc_check_shape(ctypes.byref(cs))


def n_special(shape):
    return shape.zero_expert_num + shape.copy_expert_num + shape.const_expert_num


def rank_capacity(shape):
    """Smallest per-rank receive window A of the fixed-capacity layout."""
    cs = _cs(shape)
    return lib().orc_rank_capacity(ctypes.byref(cs))


def layout(shape, topk_idx, mask=None, rank_stride=0):
    """Routing layout; returns a dict of numpy arrays plus 'status' (bit 1: a bad id was
    dropped; bit 2: a copy overflowed its rank window).  rank_stride > 0 places rank r's
    rows in [r * rank_stride, (r + 1) * rank_stride)."""
    T, K, E, P = shape.num_tokens, shape.topk, shape.num_experts, shape.num_ranks
    topk_idx = _arr(topk_idx, np.int32).reshape(T, K)
    mask = _arr(mask, np.uint8)
    cap = P * rank_stride if rank_stride > 0 else T * K
    out = dict(
        num_tokens_per_expert=np.zeros(E, np.int32),
        expert_offsets=np.zeros(E + 1, np.int32),
        recv_counts=np.zeros((E, P), np.int32),
        special_counts=np.zeros(max(n_special(shape), 1), np.int32),
        num_tokens_per_rank=np.zeros(P, np.int32),
        rank_offsets=np.zeros(P + 1, np.int32),
        is_token_in_rank=np.zeros((T, P), np.uint8),
        dst_row=np.full((T, K), -1, np.int32),
        src_info=np.full(max(cap, 1), -1, np.int32),
    )
    cs = _cs(shape)
    st = lib().orc_layout_ex(
        ctypes.byref(cs), int(rank_stride), _ptr(topk_idx), _ptr(mask),
        _ptr(out["num_tokens_per_expert"]), _ptr(out["expert_offsets"]), _ptr(out["recv_counts"]),
        _ptr(out["special_counts"]), _ptr(out["num_tokens_per_rank"]), _ptr(out["rank_offsets"]),
        _ptr(out["is_token_in_rank"]), _ptr(out["dst_row"]), _ptr(out["src_info"]),
    )
    out["special_counts"] = out["special_counts"][: n_special(shape)]
    n = int(out["expert_offsets"][E])
    out["num_rows"] = n
    out["rank_stride"] = int(rank_stride)
    if rank_stride <= 0:
        out["src_info"] = out["src_info"][:n]
    out["status"] = st
    return out


def quant_token(x_bf16, scales=None):
    """Dynamic int8 quantization of one bf16 row; returns (q int8[H], scale float32)."""
    x = _arr(x_bf16, np.uint16).ravel()
    s = _arr(scales, np.float32)
    q = np.zeros(x.size, np.int8)
    sc = np.zeros(1, np.float32)
    lib().orc_quant_token(x.size, _ptr(x), _ptr(s), _ptr(q), _ptr(sc))
    return q, sc[0]


def quant_static(x_bf16, scales=None):
    x = _arr(x_bf16, np.uint16).ravel()
    s = _arr(scales, np.float32)
    q = np.zeros(x.size, np.int8)
    lib().orc_quant_static(x.size, _ptr(x), _ptr(s), _ptr(q))
    return q


def dispatch(shape, quant_mode, x, lay, smooth=None, smooth_rows=None, weights=None, topk_idx=None):
    """Scatter of routed token copies into expert-major receive rows [N, H].

    Returns dict(expand_x (uint16 bf16 bits or int8), dynamic_scales, expand_weights)."""
    T, H, K = shape.num_tokens, shape.hidden, shape.topk
    n = lay["num_rows"] if lay.get("rank_stride", 0) <= 0 else shape.num_ranks * lay["rank_stride"]
    x = _arr(x, np.uint16).reshape(T, H)
    smooth = _arr(smooth, np.float32)
    if smooth_rows is None:
        smooth_rows = 0 if smooth is None else (1 if smooth.size == H else shape.num_experts)
    weights = _arr(weights, np.float32)
    if topk_idx is None:
        topk_idx = np.zeros((T, K), np.int32)
    topk_idx = _arr(topk_idx, np.int32)
    dst_row = _arr(lay["dst_row"], np.int32)
    rows = max(n, 1)
    ex = np.zeros((rows, H), np.uint16 if quant_mode == 0 else np.int8)
    ds = np.zeros(rows, np.float32)
    ew = np.zeros(rows, np.float32)
    cs = _cs(shape)
    st = lib().orc_dispatch(
        ctypes.byref(cs), quant_mode, _ptr(x), _ptr(smooth), smooth_rows, _ptr(weights),
        _ptr(topk_idx), _ptr(dst_row), _ptr(ex), _ptr(ds), _ptr(ew),
    )
    if st != 0:
        raise ValueError(f"oracle dispatch rejected its arguments ({st})")
    return dict(expand_x=ex[:n], dynamic_scales=ds[:n], expand_weights=ew[:n])


def combine(shape, expert_out, topk_idx, weights, lay, mask=None, ori_x=None,
            alpha1=None, alpha2=None, const_v=None):
    """Top-k weighted combine with special experts; returns float64 [T, H] (not rounded)."""
    T, H, K = shape.num_tokens, shape.hidden, shape.topk
    y = _arr(expert_out, np.uint16)
    if y is None or y.size == 0:
        y = np.zeros((1, H), np.uint16)
    out = np.zeros((T, H), np.float64)
    cs = _cs(shape)
    st = lib().orc_combine(
        ctypes.byref(cs), _ptr(y), _ptr(_arr(topk_idx, np.int32)), _ptr(_arr(weights, np.float32)),
        _ptr(_arr(mask, np.uint8)), _ptr(_arr(lay["dst_row"], np.int32)), _ptr(_arr(ori_x, np.uint16)),
        _ptr(_arr(alpha1, np.uint16)), _ptr(_arr(alpha2, np.uint16)), _ptr(_arr(const_v, np.uint16)),
        _ptr(out),
    )
    return out


def double_to_bf16(a):
    """Round float64 values to bf16 bit patterns (nearest, ties to even)."""
    a = np.asarray(a, np.float64)
    f = lib().orc_double_to_bf16
    return np.array([f(float(v)) for v in a.ravel()], np.uint16).reshape(a.shape)
