"""GPU tests of masked-row packing (the mask prologue's compact list of kept
rows), of the one-call path's dW-group budget and of the autograd wrappers'
output finish.

Packing gathers the kept rows of a mask (sequence packing leaves prompt spans
masked: "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
Fused Chunked KL Loss", abstract) so that masked rows cost no matrix work; the
results are scattered back.  Checks:
  * against the fp64 oracle on packed-document slices of the 201,088-token
    vocabulary workload, both call paths;
  * against the unpacked computation: every per-row quantity of a kept row
    (LSE, row loss, dH row) is computed by the same arithmetic in the same
    order whichever tile the row lands in, so they agree bit for bit; dW sums
    the kept rows in another grouping (fp32 rounding only);
  * masked rows give exact zeros; a bad teacher index in a masked row is not
    reported when packing (those rows are never read) and is without it.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import make_inputs
from tests.gpu_harness import TOL, max_rel, run_gpu, run_gpu_fused, say

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(cfg, T, seed=0):
    key = (cfg, T, seed)
    if key not in _cache:
        _cache[key] = make_inputs(cfg, seed=seed, T=T)
    return _cache[key]


def check_vs_oracle(x, got, ref, tol=TOL["bf16"]):
    keep = ref["keep"]
    assert abs(got["loss"] - ref["loss"]) <= tol["loss_rel"] * abs(ref["loss"])
    np.testing.assert_allclose(got["lse"][keep], ref["lse"][keep], rtol=0, atol=2e-3)
    np.testing.assert_allclose(got["row_loss"][keep], ref["row_loss"][keep], rtol=tol["loss_rel"],
                               atol=tol["loss_rel"] * np.abs(ref["row_loss"][keep]).mean())
    assert (got["lse"][~keep] == 0).all() and (got["row_loss"][~keep] == 0).all()
    assert (got["dH"][~keep] == 0).all()
    assert max_rel(got["dH"], ref["dH"]) <= tol["grad_rel"]
    assert max_rel(got["dW"], ref["dW"]) <= tol["grad_rel"]


def check_packed_vs_unpacked(a, b):
    """a: packed, b: unpacked (same inputs, same call path)."""
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-6)
    for k in ("lse", "row_loss", "dH"):
        assert np.array_equal(a[k], b[k]), k
    assert max_rel(a["dW"], b["dW"]) <= 1e-5


@pytest.mark.parametrize("T,chunk", [(1500, 300), (2300, 512)])
def test_packed_two_call_vs_oracle_and_unpacked(T, chunk):
    x = inputs(4, T)
    n = int(x.mask.sum())
    say(f"case packed two-call cfg4 slice T={T} kept={n} chunk={chunk}")
    a = run_gpu(x, chunk=chunk, grad_loss=0.8)
    check_vs_oracle(x, a, oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, mask=x.mask, grad_loss=0.8, block=128))
    b = run_gpu(x, chunk=chunk, grad_loss=0.8, compact=False)
    check_packed_vs_unpacked(a, b)


@pytest.mark.parametrize("T,chunk", [(1500, 256), (2300, 512)])
def test_packed_fused_vs_oracle_and_unpacked(T, chunk):
    x = inputs(4, T)
    say(f"case packed one-call cfg4 slice T={T} kept={int(x.mask.sum())} chunk={chunk}")
    a = run_gpu_fused(x, chunk=chunk, grad_loss=0.8)
    check_vs_oracle(x, a, oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, mask=x.mask, grad_loss=0.8, block=128))
    b = run_gpu_fused(x, chunk=chunk, grad_loss=0.8, compact=False)
    check_packed_vs_unpacked(a, b)


def test_packed_fp32_and_output_dtypes():
    import torch
    x = inputs(0, 256)
    rng = np.random.default_rng(4)
    mask = (rng.random(x.T) < 0.6).astype(np.uint8)
    x = dataclasses.replace(x, mask=mask)
    ref = oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, mask=mask, grad_loss=1.3, block=64)
    say("case packed fp32 (both paths)")
    check_vs_oracle(x, run_gpu(x, chunk=64, grad_loss=1.3), ref, TOL["f32"])
    check_vs_oracle(x, run_gpu_fused(x, chunk=64, grad_loss=1.3), ref, TOL["f32"])
    y = inputs(4, 900)
    ref = oracle.kl_dense(y.H, y.W, y.idx, y.tlogit, mask=y.mask, block=128)
    say("case packed bf16 with fp32 dH and bf16 dW outputs (both paths)")
    kw = dict(dh_dtype=torch.float32, dw_dtype=torch.bfloat16, chunk=256)
    check_vs_oracle(y, run_gpu(y, **kw), ref)
    check_vs_oracle(y, run_gpu_fused(y, **kw), ref)


def test_packed_masked_row_indices_not_read():
    import chunked_kl_loss_amd as ckl
    x = inputs(4, 700)
    masked = np.nonzero(x.mask == 0)[0]
    idx = x.idx.copy()
    idx[masked[3], 5] = x.V + 17   # out of range, in a masked row
    y = dataclasses.replace(x, idx=idx)
    say("case validate: bad index in a masked row")
    run_gpu(y, validate=True, want_grads=False)      # packed: the row is never read
    with pytest.raises(ckl.CklError) as e:
        run_gpu(y, validate=True, want_grads=False, compact=False)
    assert e.value.status == 4


def test_fused_dw_group_budget():
    # one chunk per dW group (the least memory) against the default eight:
    # only the fp32 summation of dW is grouped differently
    x = inputs(1, 3000)
    say("case one-call dW group of one chunk vs the default")
    a = run_gpu_fused(x, chunk=256)
    b = run_gpu_fused(x, chunk=256, dw_group_rows=256)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_loss", "dH"):
        assert np.array_equal(a[k], b[k]), k
    assert max_rel(b["dW"], a["dW"]) <= 1e-5
    check_vs_oracle(x, b, oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, block=128))


def test_fused_autograd_rounds_once():
    # the autograd backward of the one-call path scales the fp32 gradients of
    # the loss and rounds once: H.grad equals bf16(g * dH32) exactly
    import torch

    import chunked_kl_loss_amd as ckl
    from tests.gpu_harness import to_device
    x = inputs(4, 600)
    H, W, idx, tl, m = to_device(x)
    _, _, _, dH32, dW32 = ckl.forward_backward(H, W, idx, tl, m, None, chunk=256, dh_dtype=torch.float32,
                                               dw_dtype=torch.float32)
    Hg = H.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = ckl.chunked_kl_loss(Hg, Wg, idx, tl, m, chunk=256, fused=True)
    (0.37 * loss).backward()
    g = torch.tensor(0.37, dtype=torch.float32, device=H.device)
    assert torch.equal(Hg.grad, (dH32 * g).to(torch.bfloat16))
    assert torch.equal(Wg.grad, (dW32 * g).to(torch.bfloat16))
    # no gradient wanted: the forward computes the loss alone, equal to ckl.forward's
    loss_ng = ckl.chunked_kl_loss(H, W, idx, tl, m, chunk=256, fused=True)
    loss_fwd, _, _ = ckl.forward(H, W, idx, tl, m, chunk=256)
    assert loss_ng.item() == loss_fwd.item()
    assert abs(loss_ng.item() - loss.item()) <= 1e-6 * abs(loss.item())
    # the recomputing wrapper returns only the gradients asked for
    Wg.grad = None
    Hn = H.clone()
    loss2 = ckl.chunked_kl_loss(Hn, Wg, idx, tl, m, chunk=256)
    loss2.backward()
    assert Wg.grad is not None and Hn.grad is None


def test_scale_cast_entry_point():
    import torch

    import chunked_kl_loss_amd as ckl
    rng = np.random.default_rng(2)
    src = torch.from_numpy(rng.standard_normal(4096).astype(np.float32)).cuda()
    s = torch.tensor([1.7], dtype=torch.float32, device="cuda")
    out = ckl.scale_cast(src, torch.empty(4096, dtype=torch.bfloat16, device="cuda"), s)
    assert torch.equal(out, (src * s).to(torch.bfloat16))
    out32 = ckl.scale_cast(src, torch.empty(4096, dtype=torch.float32, device="cuda"))
    assert torch.equal(out32, src)
    same = src.clone()
    ckl.scale_cast(same, same, s)  # fp32 in place
    assert torch.equal(same, src * s)
