"""ctypes binding of libckl (include/ckl.h).

Argument marshalling only: every step of the loss runs inside the HIP library.
PyTorch provides device memory and the current stream.  If libckl.so has not
been built, loading fails with an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libckl.so")

CKL_OK = 0
CKL_ERR_INVALID_ARG = 1
CKL_ERR_UNSUPPORTED = 2
CKL_ERR_WORKSPACE = 3
CKL_ERR_BAD_INDEX = 4
CKL_ERR_HIP = 5
CKL_F32 = 0
CKL_BF16 = 1
CKL_TEACHER_LOGITS = 0
CKL_TEACHER_LOGPROBS = 1

EXPORTED = (
    "ckl_workspace_size",
    "ckl_forward",
    "ckl_forward_noalloc",
    "ckl_backward",
    "ckl_backward_plan",
    "ckl_forward_backward",
    "ckl_fused_plan",
    "ckl_scale_cast",
    "ckl_shard_forward",
    "ckl_shard_combine",
    "ckl_timing_enable",
    "ckl_timing_read",
    "ckl_status_string",
    "ckl_last_error",
    "ckl_version",
)


class CklError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ckl status {status}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32),
        ("dh_dtype", ctypes.c_int32),
        ("dw_dtype", ctypes.c_int32),
        ("validate", ctypes.c_int32),
        ("teacher_form", ctypes.c_int32),
        ("v_offset", ctypes.c_int64),
        ("v_total", ctypes.c_int64),
        ("dw_group_rows", ctypes.c_int64),
        ("compact_mask", ctypes.c_int32),
        ("reserved_", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libckl.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libckl.so not found at {p}: build it with "
                           "`python -m chunked_kl_loss_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, sz, i32, i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)
    P = ctypes.POINTER(Problem)
    lib.ckl_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.ckl_workspace_size.restype = i32
    lib.ckl_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ckl_forward.restype = i32
    lib.ckl_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ckl_forward_noalloc.restype = i32
    lib.ckl_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ckl_backward.restype = i32
    lib.ckl_backward_plan.argtypes = [P, i64p]
    lib.ckl_backward_plan.restype = i32
    lib.ckl_forward_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ckl_forward_backward.restype = i32
    lib.ckl_fused_plan.argtypes = [P, i64p]
    lib.ckl_fused_plan.restype = i32
    lib.ckl_scale_cast.argtypes = [vp, vp, ctypes.c_int64, i32, vp, vp]
    lib.ckl_scale_cast.restype = i32
    lib.ckl_shard_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ckl_shard_forward.restype = i32
    lib.ckl_shard_combine.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ckl_shard_combine.restype = i32
    lib.ckl_timing_enable.argtypes = [ctypes.c_int]
    lib.ckl_timing_enable.restype = i32
    lib.ckl_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), i64p]
    lib.ckl_timing_read.restype = i32
    lib.ckl_status_string.argtypes = [i32]
    lib.ckl_status_string.restype = ctypes.c_char_p
    lib.ckl_last_error.argtypes = []
    lib.ckl_last_error.restype = ctypes.c_char_p
    lib.ckl_version.argtypes = []
    lib.ckl_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def check(status: int, lib=None) -> None:
    if status != CKL_OK:
        lib = lib or load_library()
        raise CklError(status, lib.ckl_last_error().decode())


def make_problem(T, d, V, K, chunk, in_dtype=CKL_BF16, dh_dtype=None, dw_dtype=CKL_F32, validate=False,
                 teacher_form=CKL_TEACHER_LOGITS, v_offset=0, v_total=0, dw_group_rows=0,
                 compact_mask=False) -> Problem:
    return Problem(int(T), int(d), int(V), int(K), int(chunk), int(in_dtype),
                   int(in_dtype if dh_dtype is None else dh_dtype), int(dw_dtype), int(bool(validate)),
                   int(teacher_form), int(v_offset), int(v_total), int(dw_group_rows), int(bool(compact_mask)), 0)


def workspace_size(prob: Problem, which: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    check(lib.ckl_workspace_size(ctypes.byref(prob), int(which), ctypes.byref(out)), lib)
    return int(out.value)


def backward_plan(prob: Problem):
    lib = load_library()
    out = (ctypes.c_int64 * 5)()
    check(lib.ckl_backward_plan(ctypes.byref(prob), out), lib)
    return dict(Tc=out[0], Vc=out[1], nT=out[2], nV=out[3], n_buffers=out[4])


def fused_plan(prob: Problem):
    """Row chunks, dH split-k and dW groups of ckl_forward_backward for this problem."""
    lib = load_library()
    out = (ctypes.c_int64 * 5)()
    check(lib.ckl_fused_plan(ctypes.byref(prob), out), lib)
    return dict(rows=out[0], chunks=out[1], dh_parts=out[2], part_cols=out[3], dw_group_chunks=out[4])


KERNEL_CLASSES = ("teacher_prep", "fwd_lse", "fwd_finalize", "bwd_grad", "gemm_dhdw", "g_pass", "transpose",
                  "other")


def timing_enable(on: bool = True) -> None:
    """Start (and clear) or stop the library's per-kernel event timing."""
    lib = load_library()
    check(lib.ckl_timing_enable(int(bool(on))), lib)


def timing_read() -> dict:
    """{class name: (total ms, launches)} accumulated since timing_enable()."""
    lib = load_library()
    out = {}
    for i, name in enumerate(KERNEL_CLASSES):
        ms, n = ctypes.c_double(0), ctypes.c_int64(0)
        check(lib.ckl_timing_read(i, ctypes.byref(ms), ctypes.byref(n)), lib)
        out[name] = (ms.value, n.value)
    return out


# ------------------------------------------------------------ torch layer --
def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return CKL_BF16
    if dt == torch.float32:
        return CKL_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


# Checking aid: a byte value (0..255) with which every workspace and output
# buffer the functions below allocate is filled before the library call, so
# that a result depending on memory the library should have written (the
# workspace contents on entry do not matter, outputs are overwritten) shows up:
# 0xFF makes float32 and bf16 words NaN.  None (the default): plain
# torch.empty, nothing filled.
FILL_BYTE = None


def _empty(shape, dtype, device):
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if FILL_BYTE is not None and t.numel() > 0:
        t.view(torch.uint8).fill_(int(FILL_BYTE))
    return t


def _torch_dtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == CKL_BF16 else torch.float32


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check_inputs(H, W, idx, tlogit, mask):
    torch = _torch()
    if not (H.is_cuda and W.is_cuda and idx.is_cuda and tlogit.is_cuda):
        raise ValueError("H, W, idx and tlogit must be GPU tensors")
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1] or H.dtype != W.dtype:
        raise ValueError("H [T, d] and W [V, d] must share d and dtype")
    if idx.shape != tlogit.shape or idx.dim() != 2 or idx.shape[0] != H.shape[0]:
        raise ValueError("idx and tlogit must be [T, K]")
    if idx.dtype != torch.int32 or tlogit.dtype != torch.float32:
        raise TypeError("idx must be int32 and tlogit float32")
    for name, t in (("H", H), ("W", W), ("idx", idx), ("tlogit", tlogit)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if mask is not None:
        if mask.shape != (H.shape[0],) or mask.dtype not in (torch.uint8, torch.bool) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8/bool [T] tensor")
        if not mask.is_cuda:
            raise ValueError("mask must be a GPU tensor")
    devs = {t.device for t in (H, W, idx, tlogit) + ((mask,) if mask is not None else ())}
    if len(devs) != 1:
        raise ValueError("H, W, idx, tlogit and mask must be on one device")


def _check_lse(lse, H):
    torch = _torch()
    if (not lse.is_cuda or lse.device != H.device or lse.dtype != torch.float32 or lse.shape != (H.shape[0],)
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [T] tensor on the device of H")


def _stream_ptr(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def forward(H, W, idx, tlogit, mask=None, chunk: int = 2048, validate: bool = False,
            want_row_loss: bool = False, teacher_form: int = CKL_TEACHER_LOGITS, compact_mask: bool = True):
    """Returns (loss [1] float32, lse [T] float32, row_loss [T] or None).  tlogit holds teacher logits
    (teacher_form 0) or truncated teacher log-probabilities used as given (teacher_form 1).
    compact_mask: with a mask, only the kept rows are computed (packed first)."""
    torch = _torch()
    _check_inputs(H, W, idx, tlogit, mask)
    T, d = H.shape
    V, K = W.shape[0], idx.shape[1]
    prob = make_problem(T, d, V, K, chunk, _dtype_code(H.dtype), validate=validate, teacher_form=teacher_form,
                        compact_mask=compact_mask and mask is not None)
    lib = load_library()
    ws_bytes = workspace_size(prob, 0)
    dev = H.device
    ws = _empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    loss = _empty(1, dtype=torch.float32, device=dev)
    lse = _empty(T, dtype=torch.float32, device=dev)
    row_loss = _empty(T, dtype=torch.float32, device=dev) if want_row_loss else None
    m = mask.view(torch.uint8) if mask is not None else None
    check(lib.ckl_forward(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlogit), _ptr(m),
                          _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(ws), ws_bytes, _stream_ptr(dev)), lib)
    return loss, lse, row_loss


def backward(H, W, idx, tlogit, mask, lse, grad_loss=None, chunk: int = 2048, dh_dtype=None,
             dw_dtype=None, validate: bool = False, teacher_form: int = CKL_TEACHER_LOGITS,
             v_offset: int = 0, v_total: int = 0, compact_mask: bool = True):
    """Returns (dH, dW) of grad_loss * loss (grad_loss: [1] float32 tensor or None = 1)."""
    torch = _torch()
    _check_inputs(H, W, idx, tlogit, mask)
    _check_lse(lse, H)
    T, d = H.shape
    V, K = W.shape[0], idx.shape[1]
    in_code = _dtype_code(H.dtype)
    dh_code = in_code if dh_dtype is None else _dtype_code(dh_dtype)
    dw_code = CKL_F32 if dw_dtype is None else _dtype_code(dw_dtype)
    prob = make_problem(T, d, V, K, chunk, in_code, dh_code, dw_code, validate, teacher_form, v_offset, v_total,
                        compact_mask=compact_mask and mask is not None)
    lib = load_library()
    ws_bytes = workspace_size(prob, 1)
    dev = H.device
    ws = _empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dH = _empty((T, d), dtype=_torch_dtype(dh_code), device=dev)
    dW = _empty((V, d), dtype=_torch_dtype(dw_code), device=dev)
    m = mask.view(torch.uint8) if mask is not None else None
    if grad_loss is not None:
        grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    check(lib.ckl_backward(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlogit), _ptr(m), _ptr(lse),
                           _ptr(grad_loss), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes, _stream_ptr(dev)), lib)
    return dH, dW


def forward_backward(H, W, idx, tlogit, mask=None, grad_loss=None, chunk: int = 2048, dh_dtype=None,
                     dw_dtype=None, validate: bool = False, want_row_loss: bool = False,
                     teacher_form: int = CKL_TEACHER_LOGITS, compact_mask: bool = True, dw_group_rows: int = 0):
    """One call, no logit recompute: returns (loss [1], lse [T], row_loss [T] or None, dH, dW), the
    gradients being those of grad_loss * loss (grad_loss: [1] float32 tensor or None = 1).
    dw_group_rows: rows of logit gradients kept per dW update (0 = the library default)."""
    torch = _torch()
    _check_inputs(H, W, idx, tlogit, mask)
    T, d = H.shape
    V, K = W.shape[0], idx.shape[1]
    in_code = _dtype_code(H.dtype)
    dh_code = in_code if dh_dtype is None else _dtype_code(dh_dtype)
    dw_code = CKL_F32 if dw_dtype is None else _dtype_code(dw_dtype)
    prob = make_problem(T, d, V, K, chunk, in_code, dh_code, dw_code, validate, teacher_form,
                        dw_group_rows=dw_group_rows, compact_mask=compact_mask and mask is not None)
    lib = load_library()
    ws_bytes = workspace_size(prob, 2)
    dev = H.device
    ws = _empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    loss = _empty(1, dtype=torch.float32, device=dev)
    lse = _empty(T, dtype=torch.float32, device=dev)
    row_loss = _empty(T, dtype=torch.float32, device=dev) if want_row_loss else None
    dH = _empty((T, d), dtype=_torch_dtype(dh_code), device=dev)
    dW = _empty((V, d), dtype=_torch_dtype(dw_code), device=dev)
    m = mask.view(torch.uint8) if mask is not None else None
    if grad_loss is not None:
        grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    check(lib.ckl_forward_backward(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlogit), _ptr(m),
                                   _ptr(grad_loss), _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(dH), _ptr(dW),
                                   _ptr(ws), ws_bytes, _stream_ptr(dev)), lib)
    return loss, lse, row_loss, dH, dW


def shard_forward(H, W_shard, idx, tlogit, v_offset: int, v_total: int, chunk: int = 2048,
                  validate: bool = False, teacher_form: int = CKL_TEACHER_LOGITS):
    """One vocabulary shard (rows [v_offset, v_offset + W_shard.shape[0]) of a v_total-row head):
    returns (lse_part [T], cross_part [T]) float32."""
    torch = _torch()
    _check_inputs(H, W_shard, idx, tlogit, None)
    T, d = H.shape
    V, K = W_shard.shape[0], idx.shape[1]
    prob = make_problem(T, d, V, K, chunk, _dtype_code(H.dtype), validate=validate, teacher_form=teacher_form,
                        v_offset=v_offset, v_total=v_total)
    lib = load_library()
    ws_bytes = workspace_size(prob, 0)
    dev = H.device
    ws = _empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    lse_part = _empty(T, dtype=torch.float32, device=dev)
    cross_part = _empty(T, dtype=torch.float32, device=dev)
    check(lib.ckl_shard_forward(ctypes.byref(prob), _ptr(H), _ptr(W_shard), _ptr(idx), _ptr(tlogit),
                                _ptr(lse_part), _ptr(cross_part), _ptr(ws), ws_bytes, _stream_ptr(dev)), lib)
    return lse_part, cross_part


def shard_combine(lse_parts, cross_parts, idx, tlogit, mask=None, v_total: int = 1, d: int = 8,
                  teacher_form: int = CKL_TEACHER_LOGITS, want_row_loss: bool = False):
    """Merge [n_shards, T] partials: returns (loss [1], lse [T], row_loss [T] or None)."""
    torch = _torch()
    n_shards, T = lse_parts.shape
    K = idx.shape[1]
    for name, t in (("lse_parts", lse_parts), ("cross_parts", cross_parts), ("idx", idx), ("tlogit", tlogit)):
        if not t.is_cuda or not t.is_contiguous() or t.device != lse_parts.device:
            raise ValueError(f"{name} must be a contiguous GPU tensor on the device of lse_parts")
    if (cross_parts.shape != lse_parts.shape or lse_parts.dtype != torch.float32 or cross_parts.dtype != torch.float32
            or idx.shape != tlogit.shape or idx.shape[0] != T or idx.dtype != torch.int32
            or tlogit.dtype != torch.float32):
        raise ValueError("lse_parts, cross_parts: float32 [n_shards, T]; idx int32 and tlogit float32 [T, K]")
    if mask is not None and (mask.shape != (T,) or mask.dtype not in (torch.uint8, torch.bool) or not mask.is_cuda
                             or not mask.is_contiguous() or mask.device != lse_parts.device):
        raise ValueError("mask must be a contiguous uint8/bool [T] tensor on the device of lse_parts")
    prob = make_problem(T, d, v_total, K, 1, CKL_F32, teacher_form=teacher_form)
    lib = load_library()
    ws_bytes = workspace_size(prob, 3)
    dev = lse_parts.device
    ws = _empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    loss = _empty(1, dtype=torch.float32, device=dev)
    lse = _empty(T, dtype=torch.float32, device=dev)
    row_loss = _empty(T, dtype=torch.float32, device=dev) if want_row_loss else None
    m = mask.view(torch.uint8) if mask is not None else None
    check(lib.ckl_shard_combine(ctypes.byref(prob), int(n_shards), _ptr(lse_parts), _ptr(cross_parts), _ptr(idx),
                                _ptr(tlogit), _ptr(m), _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(ws), ws_bytes,
                                _stream_ptr(dev)), lib)
    return loss, lse, row_loss


def scale_cast(src, dst, scale=None):
    """dst = scale * src rounded once to dst's dtype (src float32; dst float32 or bfloat16, same number
    of elements; scale: [1] float32 tensor or None = 1).  Returns dst."""
    torch = _torch()
    if not (src.is_cuda and dst.is_cuda) or src.dtype != torch.float32 or src.numel() != dst.numel():
        raise ValueError("src must be a float32 GPU tensor with as many elements as dst")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    lib = load_library()
    if scale is not None:
        scale = scale.to(device=src.device, dtype=torch.float32).contiguous()
    check(lib.ckl_scale_cast(_ptr(src), _ptr(dst), int(src.numel()), _dtype_code(dst.dtype), _ptr(scale),
                             _stream_ptr(src.device)), lib)
    return dst
