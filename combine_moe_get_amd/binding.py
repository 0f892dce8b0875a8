"""ctypes binding of libmoe_get (include/moe_get.h): argument marshalling only.

Every step runs in the HIP kernels behind the C ABI; this module checks
tensor dtypes/devices, allocates outputs with PyTorch when the caller does not
pass them, and hands raw device pointers and the current HIP stream to the
library.  There is no CPU fallback: without the built library every call
raises.
"""
import ctypes
import os
from collections import namedtuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_get.so")

MOE_OK = 0
QUANT_NONE, QUANT_STATIC_INT8, QUANT_DYNAMIC_INT8 = 0, 1, 2
DEV_STATUS_BAD_EXPERT_ID = 1
DEV_STATUS_RANK_OVERFLOW = 2


class Shape(ctypes.Structure):
    """moe_get_shape_t."""
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("zero_expert_num", ctypes.c_int32),
        ("copy_expert_num", ctypes.c_int32),
        ("const_expert_num", ctypes.c_int32),
        ("num_max_dispatch_tokens_per_rank", ctypes.c_int32),
    ]

    @property
    def n_special(self):
        return self.zero_expert_num + self.copy_expert_num + self.const_expert_num

    def __repr__(self):
        return "Shape(" + ", ".join(f"{f}={getattr(self, f)}" for f, _ in self._fields_) + ")"


def make_shape(T, H, K, E, P, Z=0, C=0, Kc=0, num_max=0):
    return Shape(int(T), int(H), int(K), int(E), int(P), int(Z), int(C), int(Kc), int(num_max))


class MoeGetError(RuntimeError):
    def __init__(self, what, status):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class PreparedCall:
    """One library call with its arguments checked and marshalled once.  Calling it
    issues the C call on the current (or given) stream with no per-call checks: the
    tensors it was prepared with must stay alive and keep their shapes."""

    __slots__ = ("_fn", "_args", "_what", "_keep", "result")

    def __init__(self, fn, args, what, keep, result):
        self._fn, self._args, self._what, self._keep, self.result = fn, list(args), what, keep, result

    def __call__(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        self._args[-1] = ctypes.c_void_p(s.cuda_stream)
        st = self._fn(*self._args)
        if st != MOE_OK:
            raise MoeGetError(self._what, st)
        return self.result


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        V, I32, SZ, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int64
        SP = ctypes.POINTER(Shape)
        L.moe_get_abi_version.argtypes = []
        L.moe_get_abi_version.restype = ctypes.c_int
        L.moe_get_status_string.argtypes = [ctypes.c_int]
        L.moe_get_status_string.restype = ctypes.c_char_p
        L.moe_get_check_shape.argtypes = [SP]
        L.moe_get_check_shape.restype = ctypes.c_int
        L.moe_get_recv_capacity.argtypes = [SP]
        L.moe_get_recv_capacity.restype = I64
        L.moe_get_workspace_size.argtypes = [SP]
        L.moe_get_workspace_size.restype = SZ
        L.moe_get_layout.argtypes = [SP] + [V] * 12 + [V, SZ, V]
        L.moe_get_layout.restype = ctypes.c_int
        L.moe_get_layout_ex.argtypes = [SP, I64] + [V] * 12 + [V, SZ, V]
        L.moe_get_layout_ex.restype = ctypes.c_int
        L.moe_get_layout_noalloc.argtypes = [SP, I64] + [V] * 12 + [V]
        L.moe_get_layout_noalloc.restype = ctypes.c_int
        L.moe_get_noalloc_scratch_bytes.argtypes = []
        L.moe_get_noalloc_scratch_bytes.restype = SZ
        L.moe_get_rank_capacity.argtypes = [SP]
        L.moe_get_rank_capacity.restype = I64
        L.moe_get_layout_launches.argtypes = [SP]
        L.moe_get_layout_launches.restype = ctypes.c_int
        L.moe_layout_dispatch.argtypes = [SP, I64, I32, V, V, V, V, I32, V] + [V] * 12 + [V, V, SZ, V]
        L.moe_layout_dispatch.restype = ctypes.c_int
        L.moe_layout_dispatch_launches.argtypes = [SP, ctypes.c_int32]
        L.moe_layout_dispatch_launches.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [SP, I32, V, V, I32, V, V, V, V, V, V, V]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch_capped.argtypes = [SP, I32, I32, V, V, I32, V, V, V, V, V, V, V]
        L.moe_dispatch_capped.restype = ctypes.c_int
        L.moe_combine.argtypes = [SP] + [V] * 11
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine_capped.argtypes = [SP, I32] + [V] * 11
        L.moe_combine_capped.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().moe_get_status_string(int(status)).decode()


def abi_version():
    return lib().moe_get_abi_version()


def check_shape(shape):
    return lib().moe_get_check_shape(ctypes.byref(shape))


def recv_capacity(shape):
    return lib().moe_get_recv_capacity(ctypes.byref(shape))


def workspace_size(shape):
    return lib().moe_get_workspace_size(ctypes.byref(shape))


def rank_capacity(shape):
    """Smallest per-rank receive window of the fixed-capacity layout (moe_get_rank_capacity)."""
    return lib().moe_get_rank_capacity(ctypes.byref(shape))


def layout_launches(shape):
    """Kernel launches moe_get_layout makes for this shape (moe_get_layout_launches)."""
    n = lib().moe_get_layout_launches(ctypes.byref(shape))
    if n < 0:
        raise MoeGetError("moe_get_layout_launches", n)
    return n


def layout_dispatch_launches(shape, quant_mode):
    """Kernel launches moe_layout_dispatch makes for this shape and quant mode
    (moe_layout_dispatch_launches)."""
    n = lib().moe_layout_dispatch_launches(ctypes.byref(shape), int(quant_mode))
    if n < 0:
        raise MoeGetError("moe_layout_dispatch_launches", n)
    return n


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, name, dtypes, numel=None, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


BF16 = (torch.bfloat16,)
I32 = (torch.int32,)
F32 = (torch.float32,)
U8 = (torch.uint8, torch.bool)

Layout = namedtuple("Layout", [
    "num_tokens_per_expert", "expert_offsets", "recv_counts", "special_counts",
    "num_tokens_per_rank", "rank_offsets", "is_token_in_rank", "dst_row", "src_info", "status",
])


def alloc_layout(shape, device, rank_stride=0):
    T, K, E, P = shape.num_tokens, shape.topk, shape.num_experts, shape.num_ranks
    rows = P * rank_stride if rank_stride > 0 else T * K
    i32 = dict(dtype=torch.int32, device=device)
    return Layout(
        num_tokens_per_expert=torch.empty(E, **i32),
        expert_offsets=torch.empty(E + 1, **i32),
        recv_counts=torch.empty((E, P), **i32),
        special_counts=torch.empty(shape.n_special, **i32),
        num_tokens_per_rank=torch.empty(P, **i32),
        rank_offsets=torch.empty(P + 1, **i32),
        is_token_in_rank=torch.empty((T, P), dtype=torch.uint8, device=device),
        dst_row=torch.empty((T, K), **i32),
        src_info=torch.empty(max(rows, 1), **i32),
        status=torch.zeros(1, **i32),
    )


def alloc_workspace(shape, device):
    n = workspace_size(shape)
    if n == 0:
        raise MoeGetError("workspace", check_shape(shape))
    return torch.empty(n, dtype=torch.uint8, device=device)


def prepare_layout(shape, topk_idx, x_active_mask=None, out=None, workspace=None, rank_stride=0):
    """Checked, marshalled moe_get_layout_ex call; see layout()."""
    st = check_shape(shape)
    if st != MOE_OK:
        raise MoeGetError("layout", st)
    T, K = shape.num_tokens, shape.topk
    dev = topk_idx.device
    out = out if out is not None else alloc_layout(shape, dev, rank_stride)
    workspace = workspace if workspace is not None else alloc_workspace(shape, dev)
    rows = shape.num_ranks * rank_stride if rank_stride > 0 else T * K
    args = [
        ctypes.byref(shape), ctypes.c_int64(int(rank_stride)),
        _ptr(topk_idx, "topk_idx", I32, T * K),
        _ptr(x_active_mask, "x_active_mask", U8, T, required=False),
        _ptr(out.num_tokens_per_expert, "num_tokens_per_expert", I32, shape.num_experts),
        _ptr(out.expert_offsets, "expert_offsets", I32, shape.num_experts + 1),
        _ptr(out.recv_counts, "recv_counts", I32, shape.num_experts * shape.num_ranks),
        _ptr(out.special_counts, "special_counts", I32, shape.n_special, required=shape.n_special > 0),
        _ptr(out.num_tokens_per_rank, "num_tokens_per_rank", I32, shape.num_ranks),
        _ptr(out.rank_offsets, "rank_offsets", I32, shape.num_ranks + 1),
        _ptr(out.is_token_in_rank, "is_token_in_rank", U8, T * shape.num_ranks),
        _ptr(out.dst_row, "dst_row", I32, T * K),
        _ptr(out.src_info, "src_info", I32, rows),
        _ptr(out.status, "status", I32, 1),
        _ptr(workspace, "workspace", (torch.uint8,)),
        ctypes.c_size_t(workspace.numel()),
        None,
    ]
    return PreparedCall(lib().moe_get_layout_ex, args, "moe_get_layout",
                        (shape, topk_idx, x_active_mask, workspace), out)


def noalloc_scratch_bytes():
    """Bytes of the static device scratch behind moe_get_layout_noalloc."""
    return lib().moe_get_noalloc_scratch_bytes()


def prepare_layout_noalloc(shape, topk_idx, x_active_mask=None, out=None, rank_stride=0):
    """Checked, marshalled moe_get_layout_noalloc call (no workspace argument); see
    layout_noalloc().  `out` must be given by callers that cannot allocate."""
    st = check_shape(shape)
    if st != MOE_OK:
        raise MoeGetError("layout_noalloc", st)
    T, K = shape.num_tokens, shape.topk
    out = out if out is not None else alloc_layout(shape, topk_idx.device, rank_stride)
    rows = shape.num_ranks * rank_stride if rank_stride > 0 else T * K
    args = [
        ctypes.byref(shape), ctypes.c_int64(int(rank_stride)),
        _ptr(topk_idx, "topk_idx", I32, T * K),
        _ptr(x_active_mask, "x_active_mask", U8, T, required=False),
        _ptr(out.num_tokens_per_expert, "num_tokens_per_expert", I32, shape.num_experts),
        _ptr(out.expert_offsets, "expert_offsets", I32, shape.num_experts + 1),
        _ptr(out.recv_counts, "recv_counts", I32, shape.num_experts * shape.num_ranks),
        _ptr(out.special_counts, "special_counts", I32, shape.n_special, required=shape.n_special > 0),
        _ptr(out.num_tokens_per_rank, "num_tokens_per_rank", I32, shape.num_ranks),
        _ptr(out.rank_offsets, "rank_offsets", I32, shape.num_ranks + 1),
        _ptr(out.is_token_in_rank, "is_token_in_rank", U8, T * shape.num_ranks),
        _ptr(out.dst_row, "dst_row", I32, T * K),
        _ptr(out.src_info, "src_info", I32, rows),
        _ptr(out.status, "status", I32, 1),
        None,
    ]
    return PreparedCall(lib().moe_get_layout_noalloc, args, "moe_get_layout_noalloc",
                        (shape, topk_idx, x_active_mask), out)


def layout_noalloc(shape, topk_idx, x_active_mask=None, out=None, stream=None, rank_stride=0):
    """moe_get_layout_noalloc: the layout of layout(), its workspace in the library's static
    device scratch (no allocation in the library; raises MoeGetError with status -6 when the
    shape needs more than noalloc_scratch_bytes())."""
    return prepare_layout_noalloc(shape, topk_idx, x_active_mask, out, rank_stride)(stream)


def layout(shape, topk_idx, x_active_mask=None, out=None, workspace=None, stream=None, rank_stride=0):
    """moe_get_layout (rank_stride 0) or moe_get_layout_ex.  Returns a Layout of device
    tensors; `status` is a sticky int32 word (bit 1: an out-of-range expert id was dropped;
    bit 2: a copy did not fit its rank window)."""
    return prepare_layout(shape, topk_idx, x_active_mask, out, workspace, rank_stride)(stream)


def prepare_dispatch(shape, quant_mode, x, dst_row, x_smooth_scale=None, topk_weights=None, topk_idx=None,
                     expand_x=None, dynamic_scales=None, expand_weights=None, rows=None, max_workgroups=0):
    """Checked, marshalled moe_dispatch call (moe_dispatch_capped when max_workgroups > 0); see
    dispatch()."""
    T, H, K, E = shape.num_tokens, shape.hidden, shape.topk, shape.num_experts
    if x is None or dst_row is None:
        raise ValueError("x and dst_row are required")
    cap = max(T * K if rows is None else int(rows), 1)
    dev = x.device
    if expand_x is None:
        expand_x = torch.empty((cap, H), dtype=torch.bfloat16 if quant_mode == 0 else torch.int8, device=dev)
    if quant_mode == QUANT_DYNAMIC_INT8 and dynamic_scales is None:
        dynamic_scales = torch.empty(cap, dtype=torch.float32, device=dev)
    smooth_rows = 0
    if x_smooth_scale is not None:
        smooth_rows = 1 if x_smooth_scale.numel() == H else x_smooth_scale.numel() // H
        if smooth_rows * H != x_smooth_scale.numel() or smooth_rows not in (1, E):
            raise ValueError("x_smooth_scale must hold [H] or [num_experts, H] floats")
    args = [
        ctypes.byref(shape), int(quant_mode),
        _ptr(x, "x", BF16, T * H),
        _ptr(x_smooth_scale, "x_smooth_scale", F32, required=False),
        smooth_rows,
        _ptr(topk_weights, "topk_weights", F32, T * K, required=False),
        _ptr(topk_idx, "topk_idx", I32, T * K, required=False),
        _ptr(dst_row, "dst_row", I32, T * K),
        _ptr(expand_x, "expand_x", BF16 if quant_mode == 0 else (torch.int8,), cap * H),
        _ptr(dynamic_scales, "dynamic_scales", F32, cap, required=False),
        _ptr(expand_weights, "expand_weights", F32, cap, required=False),
        None,
    ]
    keep = (shape, x, dst_row, x_smooth_scale, topk_weights, topk_idx)
    if int(max_workgroups) != 0:  # negative: the library refuses it
        return PreparedCall(lib().moe_dispatch_capped, args[:1] + [int(max_workgroups)] + args[1:],
                            "moe_dispatch_capped", keep, (expand_x, dynamic_scales, expand_weights))
    return PreparedCall(lib().moe_dispatch, args, "moe_dispatch", keep,
                        (expand_x, dynamic_scales, expand_weights))


def dispatch(shape, quant_mode, x, dst_row, x_smooth_scale=None, topk_weights=None, topk_idx=None,
             expand_x=None, dynamic_scales=None, expand_weights=None, stream=None, rows=None, max_workgroups=0):
    """moe_dispatch.  Returns (expand_x [rows, H], dynamic_scales [rows] or None,
    expand_weights [rows] or None); rows not named by dst_row are left as they were.
    `rows` (default T * K) sizes the outputs allocated here; a fixed-capacity layout
    needs P * rank_stride.  max_workgroups > 0 caps the grid (moe_dispatch_capped)."""
    return prepare_dispatch(shape, quant_mode, x, dst_row, x_smooth_scale, topk_weights, topk_idx,
                            expand_x, dynamic_scales, expand_weights, rows, max_workgroups)(stream)


def prepare_combine(shape, expert_out, topk_idx, topk_weights, dst_row, x_active_mask=None, ori_x=None,
                    const_alpha1=None, const_alpha2=None, const_v=None, out=None, rows=None, max_workgroups=0):
    """Checked, marshalled moe_combine call (moe_combine_capped when max_workgroups > 0); see
    combine()."""
    T, H, K = shape.num_tokens, shape.hidden, shape.topk
    special = shape.copy_expert_num + shape.const_expert_num > 0
    kc = shape.const_expert_num
    rows = T * K if rows is None else int(rows)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=topk_idx.device)
    args = [
        ctypes.byref(shape),
        _ptr(expert_out, "expert_out", BF16, rows * H, required=T > 0),
        _ptr(topk_idx, "topk_idx", I32, T * K),
        _ptr(topk_weights, "topk_weights", F32, T * K),
        _ptr(x_active_mask, "x_active_mask", U8, T, required=False),
        _ptr(dst_row, "dst_row", I32, T * K),
        _ptr(ori_x, "ori_x", BF16, T * H, required=special and T > 0),
        _ptr(const_alpha1, "const_alpha1", BF16, kc * H, required=kc > 0 and T > 0),
        _ptr(const_alpha2, "const_alpha2", BF16, kc * H, required=kc > 0 and T > 0),
        _ptr(const_v, "const_v", BF16, kc * H, required=kc > 0 and T > 0),
        _ptr(out, "out", BF16, T * H),
        None,
    ]
    keep = (shape, expert_out, topk_idx, topk_weights, dst_row, x_active_mask, ori_x, const_alpha1,
            const_alpha2, const_v)
    if int(max_workgroups) != 0:  # negative: the library refuses it
        return PreparedCall(lib().moe_combine_capped, args[:1] + [int(max_workgroups)] + args[1:],
                            "moe_combine_capped", keep, out)
    return PreparedCall(lib().moe_combine, args, "moe_combine", keep, out)


def combine(shape, expert_out, topk_idx, topk_weights, dst_row, x_active_mask=None, ori_x=None,
            const_alpha1=None, const_alpha2=None, const_v=None, out=None, stream=None, rows=None,
            max_workgroups=0):
    """moe_combine.  Returns out [T, H] bf16.  `rows` is the number of receive rows expert_out
    must hold (default T * K, which covers every compact layout; a fixed-capacity layout needs
    P * rank_stride; a caller that knows N may pass rows=N).  max_workgroups > 0 caps the grid
    (moe_combine_capped)."""
    return prepare_combine(shape, expert_out, topk_idx, topk_weights, dst_row, x_active_mask, ori_x,
                           const_alpha1, const_alpha2, const_v, out, rows, max_workgroups)(stream)


def _smooth_rows(shape, x_smooth_scale):
    H, E = shape.hidden, shape.num_experts
    if x_smooth_scale is None:
        return 0
    n = 1 if x_smooth_scale.numel() == H else x_smooth_scale.numel() // H
    if n * H != x_smooth_scale.numel() or n not in (1, E):
        raise ValueError("x_smooth_scale must hold [H] or [num_experts, H] floats")
    return n


def prepare_layout_dispatch(shape, quant_mode, x, topk_idx, x_active_mask=None, x_smooth_scale=None,
                            topk_weights=None, out=None, expand_x=None, dynamic_scales=None, expand_weights=None,
                            workspace=None, rank_stride=0):
    """Checked, marshalled moe_layout_dispatch call; see layout_dispatch()."""
    st = check_shape(shape)
    if st != MOE_OK:
        raise MoeGetError("layout_dispatch", st)
    T, H, K, E, P = shape.num_tokens, shape.hidden, shape.topk, shape.num_experts, shape.num_ranks
    dev = topk_idx.device
    rows = P * rank_stride if rank_stride > 0 else T * K
    cap = max(rows, 1)
    out = out if out is not None else alloc_layout(shape, dev, rank_stride)
    workspace = workspace if workspace is not None else alloc_workspace(shape, dev)
    if expand_x is None:
        expand_x = torch.empty((cap, H), dtype=torch.bfloat16 if quant_mode == 0 else torch.int8, device=dev)
    if quant_mode == QUANT_DYNAMIC_INT8 and dynamic_scales is None:
        dynamic_scales = torch.empty(cap, dtype=torch.float32, device=dev)
    args = [
        ctypes.byref(shape), ctypes.c_int64(int(rank_stride)), int(quant_mode),
        _ptr(topk_idx, "topk_idx", I32, T * K),
        _ptr(x_active_mask, "x_active_mask", U8, T, required=False),
        _ptr(x, "x", BF16, T * H),
        _ptr(x_smooth_scale, "x_smooth_scale", F32, required=False),
        _smooth_rows(shape, x_smooth_scale),
        _ptr(topk_weights, "topk_weights", F32, T * K, required=False),
        _ptr(out.num_tokens_per_expert, "num_tokens_per_expert", I32, E),
        _ptr(out.expert_offsets, "expert_offsets", I32, E + 1),
        _ptr(out.recv_counts, "recv_counts", I32, E * P),
        _ptr(out.special_counts, "special_counts", I32, shape.n_special, required=shape.n_special > 0),
        _ptr(out.num_tokens_per_rank, "num_tokens_per_rank", I32, P),
        _ptr(out.rank_offsets, "rank_offsets", I32, P + 1),
        _ptr(out.is_token_in_rank, "is_token_in_rank", U8, T * P),
        _ptr(out.dst_row, "dst_row", I32, T * K),
        _ptr(out.src_info, "src_info", I32, rows),
        _ptr(expand_x, "expand_x", BF16 if quant_mode == 0 else (torch.int8,), rows * H),
        _ptr(dynamic_scales, "dynamic_scales", F32, rows, required=False),
        _ptr(expand_weights, "expand_weights", F32, rows, required=False),
        _ptr(out.status, "status", I32, 1),
        _ptr(workspace, "workspace", (torch.uint8,)),
        ctypes.c_size_t(workspace.numel()),
        None,
    ]
    keep = (shape, x, topk_idx, x_active_mask, x_smooth_scale, topk_weights, workspace)
    return PreparedCall(lib().moe_layout_dispatch, args, "moe_layout_dispatch", keep,
                        (out, expand_x, dynamic_scales, expand_weights))


def layout_dispatch(shape, quant_mode, x, topk_idx, x_active_mask=None, x_smooth_scale=None, topk_weights=None,
                    out=None, expand_x=None, dynamic_scales=None, expand_weights=None, workspace=None,
                    stream=None, rank_stride=0):
    """moe_layout_dispatch: layout and dispatch in one call (one kernel for T * K <= 8192
    slots; above that the layout kernels, which also read x ahead into the GPU's caches, then
    the dispatch kernel).  Returns (Layout, expand_x, dynamic_scales or None, expand_weights or
    None), identical to layout() followed by dispatch()."""
    return prepare_layout_dispatch(shape, quant_mode, x, topk_idx, x_active_mask, x_smooth_scale, topk_weights,
                                   out, expand_x, dynamic_scales, expand_weights, workspace, rank_stride)(stream)
