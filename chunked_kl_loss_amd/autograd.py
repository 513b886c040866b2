"""torch.autograd wrappers.

ChunkedKLLoss: the forward saves (H, W, idx, tlogit, mask, lse) and the
backward recomputes the logit tiles inside libckl.

FusedChunkedKLLoss: one library call in the forward computes the loss and the
gradients of the loss itself (no recompute); the backward only scales them by
the incoming gradient (1 for a loss that is backpropagated directly)."""
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
        H, W, idx, tlogit, lse, mask = ctx.saved_tensors
        mask = mask if ctx.has_mask else None
        g = grad.reshape(1).to(torch.float32)
        dH, dW = _binding.backward(H, W, idx, tlogit, mask, lse, g, chunk=ctx.chunk,
                                   dh_dtype=H.dtype, dw_dtype=W.dtype, teacher_form=ctx.teacher_form)
        return dH, dW, None, None, None, None, None


class FusedChunkedKLLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, idx, tlogit, mask=None, chunk: int = 2048, teacher_form: int = 0):
        loss, _, _, dH, dW = _binding.forward_backward(H, W, idx, tlogit, mask, None, chunk=chunk,
                                                       dh_dtype=H.dtype, dw_dtype=W.dtype,
                                                       teacher_form=teacher_form)
        ctx.save_for_backward(dH, dW)
        return loss[0]

    @staticmethod
    def backward(ctx, grad):
        dH, dW = ctx.saved_tensors
        g = grad.to(torch.float32)
        return ((dH.float() * g).to(dH.dtype), (dW.float() * g).to(dW.dtype), None, None, None, None, None)


def chunked_kl_loss(H, W, idx, tlogit, mask=None, chunk: int = 2048, fused: bool = False, teacher_form: int = 0):
    """Mean forward KL(teacher || student) over unmasked rows, differentiable
    with respect to H and W.  fused=True computes the gradients together with
    the loss (one pass over the logits, chunk x V extra workspace).
    teacher_form 1: tlogit holds truncated teacher log-probabilities, used as
    given (teacher mass below one)."""
    if fused:
        return FusedChunkedKLLoss.apply(H, W, idx, tlogit, mask, chunk, teacher_form)
    return ChunkedKLLoss.apply(H, W, idx, tlogit, mask, chunk, teacher_form)
