"""torch.autograd wrappers.

ChunkedKLLoss: the forward saves (H, W, idx, tlogit, mask, lse) and the
backward recomputes the logit tiles inside libckl.

FusedChunkedKLLoss: one library call in the forward computes the loss and the
fp32 gradients of the loss itself (no recompute); the backward multiplies them
by the incoming gradient and rounds them once to the dtypes of H and W, in the
library (ckl_scale_cast).  When neither H nor W needs a gradient the forward
computes the loss alone."""
from __future__ import annotations

import torch

from . import _binding


class ChunkedKLLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, idx, tlogit, mask=None, chunk: int = 2048, teacher_form: int = 0):
        loss, lse, _ = _binding.forward(H, W, idx, tlogit, mask, chunk=chunk, teacher_form=teacher_form)
        ctx.save_for_backward(H, W, idx, tlogit, lse, mask if mask is not None else torch.empty(0))
        ctx.has_mask = mask is not None
        ctx.chunk = chunk
        ctx.teacher_form = teacher_form
        return loss[0]

    @staticmethod
    def backward(ctx, grad):
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w):
            return None, None, None, None, None, None, None
        H, W, idx, tlogit, lse, mask = ctx.saved_tensors
        mask = mask if ctx.has_mask else None
        g = grad.reshape(1).to(torch.float32)
        dH, dW = _binding.backward(H, W, idx, tlogit, mask, lse, g, chunk=ctx.chunk,
                                   dh_dtype=H.dtype, dw_dtype=W.dtype, teacher_form=ctx.teacher_form)
        return (dH if need_h else None), (dW if need_w else None), None, None, None, None, None


class FusedChunkedKLLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, idx, tlogit, mask=None, chunk: int = 2048, teacher_form: int = 0,
                dw_group_rows: int = 0):
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        ctx.dtypes = (H.dtype, W.dtype)
        if not (need_h or need_w):
            loss, _, _ = _binding.forward(H, W, idx, tlogit, mask, chunk=chunk, teacher_form=teacher_form)
            ctx.save_for_backward(torch.empty(0, device=H.device), torch.empty(0, device=H.device))
            return loss[0]
        # gradients of the loss itself, kept in fp32 until the incoming
        # gradient is known
        loss, _, _, dH, dW = _binding.forward_backward(H, W, idx, tlogit, mask, None, chunk=chunk,
                                                       dh_dtype=torch.float32, dw_dtype=torch.float32,
                                                       teacher_form=teacher_form, dw_group_rows=dw_group_rows)
        ctx.save_for_backward(dH if need_h else torch.empty(0, device=H.device),
                              dW if need_w else torch.empty(0, device=H.device))
        return loss[0]

    @staticmethod
    def backward(ctx, grad):
        dH32, dW32 = ctx.saved_tensors
        h_dtype, w_dtype = ctx.dtypes
        g = grad.reshape(1).to(torch.float32)
        dH = dW = None
        if ctx.needs_input_grad[0]:
            dH = _binding.scale_cast(dH32, torch.empty(dH32.shape, dtype=h_dtype, device=dH32.device), g)
        if ctx.needs_input_grad[1]:
            dW = _binding.scale_cast(dW32, torch.empty(dW32.shape, dtype=w_dtype, device=dW32.device), g)
        return dH, dW, None, None, None, None, None, None


def chunked_kl_loss(H, W, idx, tlogit, mask=None, chunk: int = 2048, fused: bool = False, teacher_form: int = 0,
                    dw_group_rows: int = 0):
    """Mean forward KL(teacher || student) over unmasked rows, differentiable
    with respect to H and W.  fused=True computes the gradients together with
    the loss (one pass over the logits; it keeps the logit gradients of up to
    dw_group_rows rows, 0 = the library default of min(16384, 8 chunks), so
    a smaller value holds less memory and updates dW more often).
    teacher_form 1: tlogit holds truncated teacher log-probabilities, used as
    given (teacher mass below one).

    Leading batch dimensions are flattened into rows: H [..., d], idx and
    tlogit [..., K], mask [...].  The library takes contiguous tensors, int32
    indices and fp32 teacher values: other layouts and integer / float types
    are converted here (no copy when they already match; H and W keep their
    dtype, which selects the bf16 or fp32 path)."""
    d, K = H.shape[-1], idx.shape[-1]
    if idx.shape[:-1] != H.shape[:-1] or tlogit.shape != idx.shape or (mask is not None and mask.shape != H.shape[:-1]):
        raise ValueError("H [..., d], idx and tlogit [..., K] and mask [...] must share their leading dimensions")
    H, W = H.reshape(-1, d).contiguous(), W.contiguous()
    idx = idx.reshape(-1, K).to(torch.int32).contiguous()
    tlogit = tlogit.reshape(-1, K).to(torch.float32).contiguous()
    if mask is not None:
        mask = mask.reshape(-1).contiguous()
    if fused:
        return FusedChunkedKLLoss.apply(H, W, idx, tlogit, mask, chunk, teacher_form, dw_group_rows)
    return ChunkedKLLoss.apply(H, W, idx, tlogit, mask, chunk, teacher_form)
