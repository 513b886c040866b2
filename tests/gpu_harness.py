"""Helpers shared by the GPU tests: run the HIP library on host inputs from
``synth`` and bring the results back as float64 numpy arrays.  Imports the
product package only; the oracle is called by the tests themselves."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances (the oracle is fp64; the GPU path computes in fp32 with inputs as
# given).  bf16 inputs: loss relative error <= 2e-3 and dH / dW max-abs error
# <= 1e-2 * max|ref|.  fp32 inputs: 1e-5 relative for both.
TOL = {
    "bf16": dict(loss_rel=2e-3, grad_rel=1e-2),
    "f32": dict(loss_rel=1e-5, grad_rel=1e-5),
}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x, device="cuda"):
    import torch
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).to(device)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        H = torch.from_numpy(x.H).to(device)
        W = torch.from_numpy(x.W).to(device)
    idx = torch.from_numpy(x.idx).to(device)
    tl = torch.from_numpy(x.tlogit).to(device)
    mask = None if x.mask is None else torch.from_numpy(x.mask).to(device)
    return H, W, idx, tl, mask


def _host(t, as64):
    return t.double().cpu().numpy() if as64 else t.float().cpu().numpy()


def run_gpu(x, chunk=None, grad_loss=1.0, dh_dtype=None, dw_dtype=None, mask="inputs", validate=False,
            want_grads=True, teacher_form=0, compact=True, as64=True):
    """Forward + backward through the C ABI.  Returns float64 numpy results
    (float32 with as64=False: every GPU output is exactly representable).
    compact: with a mask, the library packs the kept rows first (else masked
    rows are computed and zeroed)."""
    import torch

    import chunked_kl_loss_amd as ckl
    H, W, idx, tl, m = to_device(x)
    if not isinstance(mask, str):
        m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=np.uint8)).cuda()
    chunk = x.chunk if chunk is None else chunk
    loss, lse, row_loss = ckl.forward(H, W, idx, tl, m, chunk=chunk, validate=validate, want_row_loss=True,
                                      teacher_form=teacher_form, compact_mask=compact)
    out = dict(loss=float(loss.item()), lse=lse.double().cpu().numpy(), row_loss=row_loss.double().cpu().numpy())
    if want_grads:
        g = torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
        dH, dW = ckl.backward(H, W, idx, tl, m, lse, g, chunk=chunk, dh_dtype=dh_dtype, dw_dtype=dw_dtype,
                              validate=validate, teacher_form=teacher_form, compact_mask=compact)
        torch.cuda.synchronize()
        out["dH"] = _host(dH, as64)
        out["dW"] = _host(dW, as64)
    del H, W, idx, tl, m
    torch.cuda.empty_cache()
    return out


def run_gpu_fused(x, chunk=None, grad_loss=1.0, dh_dtype=None, dw_dtype=None, mask="inputs", validate=False,
                  teacher_form=0, compact=True, dw_group_rows=0, as64=True):
    """The one-call forward + backward (no logit recompute) through the C ABI."""
    import torch

    import chunked_kl_loss_amd as ckl
    H, W, idx, tl, m = to_device(x)
    if not isinstance(mask, str):
        m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=np.uint8)).cuda()
    chunk = x.chunk if chunk is None else chunk
    g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    loss, lse, row_loss, dH, dW = ckl.forward_backward(H, W, idx, tl, m, g, chunk=chunk, dh_dtype=dh_dtype,
                                                       dw_dtype=dw_dtype, validate=validate, want_row_loss=True,
                                                       teacher_form=teacher_form, compact_mask=compact,
                                                       dw_group_rows=dw_group_rows)
    torch.cuda.synchronize()
    out = dict(loss=float(loss.item()), lse=lse.double().cpu().numpy(), row_loss=row_loss.double().cpu().numpy(),
               dH=_host(dH, as64), dW=_host(dW, as64))
    del H, W, idx, tl, m, dH, dW
    torch.cuda.empty_cache()
    return out


def max_rel(got, ref):
    """max |got - ref| / max |ref| (the gradient criterion)."""
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    return err / scale if scale > 0 else err
