"""GPU parity of the vocabulary-shard path: W split by rows into ragged
shards (not multiples of the 256-row tile), each shard's forward partials
(log-sum-exp over its rows and its share of the cross term) merged by
ckl_shard_combine, then the backward run per shard with the merged LSE.
Checked against the fp64 oracle on the whole problem (loss, per-row LSE and
KL, dH as the sum of the shards' contributions, dW as the concatenation of
the shards' rows) and against the unsharded library call.

Tolerances as in the other parity tests (bf16: loss 2e-3 relative, dH / dW
1e-2 of max|ref|; fp32: 1e-5); shard-vs-unsharded LSE agreement 2e-5
absolute (the merge of fp32 partials in fp64).
"""
import numpy as np
import pytest

from synth import make_inputs
from tests.gpu_harness import TOL, max_rel, run_gpu, say, to_device
from tests.test_parity_gpu import oracle_full, with_logprob_teacher

pytestmark = pytest.mark.gpu


def run_shards(x, bounds, grad_loss=1.0, chunk=None, teacher_form=0):
    import torch

    import chunked_kl_loss_amd as ckl
    H, W, idx, tl, m = to_device(x)
    chunk = x.chunk if chunk is None else chunk
    lse_parts, cross_parts = [], []
    for v0, v1 in zip(bounds[:-1], bounds[1:]):
        lp, cp = ckl.shard_forward(H, W[v0:v1].contiguous(), idx, tl, v_offset=v0, v_total=x.V, chunk=chunk,
                                   teacher_form=teacher_form)
        lse_parts.append(lp)
        cross_parts.append(cp)
    loss, lse, row_loss = ckl.shard_combine(torch.stack(lse_parts).contiguous(), torch.stack(cross_parts).contiguous(),
                                            idx, tl, m, v_total=x.V, d=x.d, teacher_form=teacher_form,
                                            want_row_loss=True)
    g = torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    dH = torch.zeros((x.T, x.d), dtype=torch.float64, device="cuda")
    dW = []
    for v0, v1 in zip(bounds[:-1], bounds[1:]):
        dh, dw = ckl.backward(H, W[v0:v1].contiguous(), idx, tl, m, lse, g, chunk=chunk, dh_dtype=torch.float32,
                              dw_dtype=torch.float32, teacher_form=teacher_form, v_offset=v0, v_total=x.V)
        dH += dh.double()   # the all-reduce of a vocabulary-parallel run
        dW.append(dw.double())
    torch.cuda.synchronize()
    return dict(loss=float(loss.item()), lse=lse.double().cpu().numpy(), row_loss=row_loss.double().cpu().numpy(),
                dH=dH.cpu().numpy(), dW=torch.cat(dW).cpu().numpy())


def check(x, got, ref, tol, lse_tol):
    keep = ref["keep"]
    assert abs(got["loss"] - ref["loss"]) <= tol["loss_rel"] * abs(ref["loss"]), (got["loss"], ref["loss"])
    np.testing.assert_allclose(got["lse"][keep], ref["lse"][keep], rtol=0, atol=lse_tol)
    np.testing.assert_allclose(got["row_loss"][keep], ref["row_loss"][keep], rtol=tol["loss_rel"],
                               atol=tol["loss_rel"] * np.abs(ref["row_loss"][keep]).mean())
    assert (got["lse"][~keep] == 0).all() and (got["row_loss"][~keep] == 0).all()
    e_h, e_w = max_rel(got["dH"], ref["dH"]), max_rel(got["dW"], ref["dW"])
    assert e_h <= tol["grad_rel"], e_h
    assert e_w <= tol["grad_rel"], e_w
    return e_h, e_w


def test_shards_fp32_tiny():
    x = make_inputs(0, seed=0)
    bounds = [0, 700, 1301, x.V]
    say(f"case shards fp32 T={x.T} V={x.V} bounds={bounds}")
    got = run_shards(x, bounds, grad_loss=0.8)
    e = check(x, got, oracle_full(x, grad_loss=0.8), TOL["f32"], 1e-5)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e}")


def test_shards_bf16_vs_oracle_and_unsharded():
    x = make_inputs(1, seed=0, T=1000)
    bounds = [0, 10000, 22345, x.V]
    say(f"case shards bf16 T={x.T} V={x.V} bounds={bounds}")
    got = run_shards(x, bounds, grad_loss=0.5, chunk=400)
    e = check(x, got, oracle_full(x, grad_loss=0.5), TOL["bf16"], 2e-3)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e}")
    whole = run_gpu(x, chunk=400, grad_loss=0.5, want_grads=False)
    assert abs(got["loss"] - whole["loss"]) <= 1e-6 * abs(whole["loss"])
    np.testing.assert_allclose(got["lse"], whole["lse"], rtol=0, atol=2e-5)


def test_shards_masked_logprob_teacher():
    x = with_logprob_teacher(make_inputs(4, seed=0, T=600))
    bounds = [0, 50000, 50001, 120000, x.V]   # includes a one-row shard
    say(f"case shards masked log-prob teacher T={x.T} bounds={bounds}")
    got = run_shards(x, bounds, chunk=256, teacher_form=1)
    check(x, got, oracle_full(x, teacher_form=1), TOL["bf16"], 2e-3)


def test_shard_validate_accepts_other_shards_indices():
    import chunked_kl_loss_amd as ckl
    x = make_inputs(1, seed=2, T=64)
    H, W, idx, tl, _ = to_device(x)
    # indices belong to [0, V); a shard of the first 1000 rows must accept all of them
    ckl.shard_forward(H, W[:1000].contiguous(), idx, tl, v_offset=0, v_total=x.V, validate=True)
    bad = idx.clone()
    bad[3, 1] = x.V   # outside the whole vocabulary
    with pytest.raises(ckl.CklError) as e:
        ckl.shard_forward(H, W[:1000].contiguous(), bad, tl, v_offset=0, v_total=x.V, validate=True)
    assert e.value.status == 4
