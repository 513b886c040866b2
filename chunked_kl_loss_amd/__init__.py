"""Fused chunked forward-KL distillation loss for AMD MI355X (gfx950).

The loss of a student output head against a sparse cached top-K teacher,
computed by hand-written HIP kernels behind the C ABI in include/ckl.h:

    loss, lse, _ = forward(H, W, idx, tlogit, mask, chunk)
    dH, dW = backward(H, W, idx, tlogit, mask, lse, grad_loss, chunk)

or, in one call without recomputing the logits,

    loss, lse, _, dH, dW = forward_backward(H, W, idx, tlogit, mask, grad_loss, chunk)

or, through autograd, ``chunked_kl_loss(H, W, idx, tlogit, mask, chunk, fused=False)``.
"""
from ._binding import (  # noqa: F401
    CKL_BF16,
    CKL_F32,
    CklError,
    Problem,
    backward,
    backward_plan,
    forward,
    forward_backward,
    fused_plan,
    scale_cast,
    load_library,
    make_problem,
    shard_combine,
    shard_forward,
    timing_enable,
    timing_read,
    workspace_size,
)
from .autograd import ChunkedKLLoss, FusedChunkedKLLoss, chunked_kl_loss  # noqa: F401
