"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Element by element on problems the oracle finishes in seconds (the tiny fp32
workload, the 4K x 32K bf16 workload, and reduced-row slices of the
201,088-vocabulary workloads with ragged row counts), and on sampled rows plus
size-independent properties at full size in the launch configuration the
benchmark times.

Tolerances: bf16 inputs -- loss relative error <= 2e-3, dH / dW max-abs error
<= 1e-2 * max|ref|; fp32 inputs -- 1e-5 relative.  Per-row log-sum-exp:
absolute error <= 2e-3 for bf16 (fp32 accumulation of d products of size
~|h||w|/d plus fp32 exponent sums; observed errors are ~1e-5) and <= 1e-5 for
fp32.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs
from tests.gpu_harness import TOL, max_rel, run_gpu, say

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(cfg, seed=0, T=None):
    key = (cfg, seed, T)
    if key not in _cache:
        _cache[key] = make_inputs(cfg, seed=seed, T=T)
    return _cache[key]


def check_full(x, got, ref, tol, lse_tol):
    keep = ref["keep"]
    assert abs(got["loss"] - ref["loss"]) <= tol["loss_rel"] * abs(ref["loss"]), (got["loss"], ref["loss"])
    np.testing.assert_allclose(got["lse"][keep], ref["lse"][keep], rtol=0, atol=lse_tol)
    np.testing.assert_allclose(got["row_loss"][keep], ref["row_loss"][keep], rtol=tol["loss_rel"],
                               atol=tol["loss_rel"] * np.abs(ref["row_loss"][keep]).mean())
    assert (got["lse"][~keep] == 0).all() and (got["row_loss"][~keep] == 0).all()
    e_h = max_rel(got["dH"], ref["dH"])
    e_w = max_rel(got["dW"], ref["dW"])
    assert e_h <= tol["grad_rel"], e_h
    assert e_w <= tol["grad_rel"], e_w
    assert (got["dH"][~keep] == 0).all()
    return e_h, e_w


def oracle_full(x, grad_loss=1.0, mask="inputs", teacher_form=0):
    m = x.mask if isinstance(mask, str) else mask
    return oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, mask=m, grad_loss=grad_loss, block=128,
                           teacher_form=teacher_form)


def with_logprob_teacher(x, seed=31, extra=400, n_neg_inf=0):
    """The same problem with the K cached values replaced by the top-K
    log-probabilities of a teacher over K + extra classes (teacher mass below
    one), optionally with some -inf entries (zero-probability tokens)."""
    rng = np.random.default_rng(seed)
    full = rng.normal(0.0, 2.0, size=(x.T, x.K + extra))
    full -= full.max(axis=1, keepdims=True)
    full -= np.log(np.exp(full).sum(axis=1, keepdims=True))
    lp = np.sort(full, axis=1)[:, ::-1][:, :x.K].astype(np.float32)
    if n_neg_inf:
        rows = rng.choice(x.T, size=n_neg_inf, replace=False)
        lp[rows, -1] = -np.inf
    return dataclasses.replace(x, tlogit=np.ascontiguousarray(lp))


# ------------------------------------------------------------- full parity --
def test_tiny_fp32_full():
    x = inputs(0)
    say(f"case tiny fp32 T={x.T} d={x.d} V={x.V} K={x.K} chunk={x.chunk}")
    got = run_gpu(x)
    ref = oracle_full(x)
    e = check_full(x, got, ref, TOL["f32"], 1e-5)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e} loss {got['loss']:.6f} ref {ref['loss']:.6f}")


def test_small_bf16_full():
    x = inputs(1)
    say(f"case small bf16 T={x.T} d={x.d} V={x.V} K={x.K} chunk={x.chunk}")
    got = run_gpu(x)
    ref = oracle_full(x)
    e = check_full(x, got, ref, TOL["bf16"], 2e-3)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e} loss {got['loss']:.6f} ref {ref['loss']:.6f}")


@pytest.mark.parametrize("cfg,T", [(2, 1000), (3, 677), (4, 677)])
def test_large_vocab_row_slices(cfg, T):
    x = inputs(cfg, T=T)
    say(f"case cfg{cfg} slice T={x.T} d={x.d} V={x.V} K={x.K} chunk={x.chunk} masked={x.mask is not None}")
    got = run_gpu(x)
    ref = oracle_full(x)
    e = check_full(x, got, ref, TOL["bf16"], 2e-3)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e} loss {got['loss']:.6f} ref {ref['loss']:.6f}")


@pytest.mark.parametrize("chunk", [1, 40, 333, 100000])
def test_chunk_sizes_multi_block(chunk):
    # small chunks force several token and vocabulary blocks in the backward
    import chunked_kl_loss_amd as ckl
    x = inputs(1, T=1000)
    plan = ckl.backward_plan(ckl.make_problem(x.T, x.d, x.V, x.K, chunk))
    say(f"case chunk={chunk} T={x.T} plan={plan}")
    got = run_gpu(x, chunk=chunk, grad_loss=0.75)
    ref = oracle_full(x, grad_loss=0.75)
    check_full(x, got, ref, TOL["bf16"], 2e-3)


def test_chunk_plans_cover_both_block_kinds():
    import chunked_kl_loss_amd as ckl
    x = inputs(1, T=1000)
    plans = [ckl.backward_plan(ckl.make_problem(x.T, x.d, x.V, x.K, c)) for c in (1, 40, 333, 100000)]
    assert any(p["nT"] > 1 for p in plans) and any(p["nV"] > 1 for p in plans)
    assert any(p["nT"] == 1 and p["nV"] == 1 for p in plans)


# ---------------------------------------------------------------- edge cases --
def _custom(T, d, V, K, dtype="bf16", seed=5, mask=None, tscale=1.0):
    from synth import Inputs, bf16_bits_to_f32, bf16_round_bits
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, d)).astype(np.float32)
    W = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    tl = (rng.normal(0, np.sqrt(2), size=(T, K)) * tscale).astype(np.float32)
    Hb = Wb = None
    if dtype == "bf16":
        Hb, Wb = bf16_round_bits(H), bf16_round_bits(W)
        H, W = bf16_bits_to_f32(Hb), bf16_bits_to_f32(Wb)
    return Inputs(T=T, d=d, V=V, K=K, chunk=64, dtype=dtype, H=H, W=W, idx=idx, tlogit=tl, mask=mask,
                  H_bits=Hb, W_bits=Wb)


@pytest.mark.parametrize("T,d,V,K,dtype", [
    (1, 8, 16, 1, "bf16"),        # one row, top-1 teacher, tiny head
    (3, 8, 1000, 7, "f32"),       # ragged vocabulary, fp32
    (130, 24, 300, 300, "bf16"),  # K = V: full-support teacher; ragged rows
    (257, 136, 129, 5, "bf16"),   # everything one past a tile boundary
    (64, 4096, 4096, 64, "bf16"), # long hidden size
    (40, 64, 5000, 4096, "bf16"), # K at its maximum (4096 teacher entries per row)
    (300, 64, 9000, 2, "bf16"),   # a short teacher list ending early in a long vocabulary walk
    (17, 16384, 700, 5, "bf16"),  # 16K hidden size (256 k slices per tile)
])
def test_edge_shapes(T, d, V, K, dtype):
    x = _custom(T, d, V, K, dtype)
    say(f"case edge T={T} d={d} V={V} K={K} {dtype}")
    got = run_gpu(x, chunk=3, grad_loss=1.5)
    ref = oracle_full(x, grad_loss=1.5)
    check_full(x, got, ref, TOL[dtype], 2e-3 if dtype == "bf16" else 1e-5)


def test_masks_all_and_one():
    x = _custom(200, 64, 700, 9)
    say("case all rows masked")
    got = run_gpu(x, mask=np.zeros(200, np.uint8))
    assert got["loss"] == 0.0
    assert (got["dH"] == 0).all() and (got["dW"] == 0).all() and (got["lse"] == 0).all()
    say("case one kept row")
    m = np.zeros(200, np.uint8)
    m[137] = 1
    got = run_gpu(x, mask=m, grad_loss=3.0)
    ref = oracle_full(x, grad_loss=3.0, mask=m)
    check_full(x, got, ref, TOL["bf16"], 2e-3)


def test_output_dtypes_bf16():
    import torch
    x = _custom(300, 96, 1500, 11)
    say("case bf16 dH and dW outputs")
    got = run_gpu(x, dh_dtype=torch.bfloat16, dw_dtype=torch.bfloat16, chunk=5)
    ref = oracle_full(x)
    check_full(x, got, ref, TOL["bf16"], 2e-3)


def test_validate_reports_bad_indices():
    import chunked_kl_loss_amd as ckl
    x = _custom(50, 16, 200, 6)
    run_gpu(x, validate=True)  # valid indices pass
    for bad in ("range", "negative", "repeat"):
        y = _custom(50, 16, 200, 6)
        if bad == "range":
            y.idx[7, 2] = 200
        elif bad == "negative":
            y.idx[3, 0] = -1
        else:
            y.idx[9, 4] = y.idx[9, 1]
        say(f"case validate {bad}")
        with pytest.raises(ckl.CklError) as e:
            run_gpu(y, validate=True, want_grads=False)
        assert e.value.status == 4
        # without validation an out-of-range entry must not fault: it matches
        # no column; the call completes
        run_gpu(y, validate=False)


def test_bitwise_deterministic():
    x = inputs(1, T=1500)
    say("case determinism")
    a = run_gpu(x, chunk=100)
    b = run_gpu(x, chunk=100)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_loss", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


def test_side_stream_matches_default_stream():
    # every launch and copy of a call goes to the caller's stream: on a
    # non-default stream (default priority) the results are those of the
    # default stream, bit for bit, for both paths
    import torch

    from tests.gpu_harness import run_gpu_fused
    x = _custom(700, 136, 3000, 40, mask=(np.arange(700) % 3 != 0).astype(np.uint8))
    say("case non-default stream")
    a, af = run_gpu(x, chunk=200), run_gpu_fused(x, chunk=200)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b, bf = run_gpu(x, chunk=200), run_gpu_fused(x, chunk=200)
    torch.cuda.synchronize()
    for r, q in ((a, b), (af, bf)):
        assert r["loss"] == q["loss"]
        for k in ("lse", "row_loss", "dH", "dW"):
            assert np.array_equal(r[k], q[k]), k


def test_binding_rejects_misplaced_tensors():
    # host tensors or mismatched arguments are refused before any launch
    import torch

    import chunked_kl_loss_amd as ckl
    from tests.gpu_harness import to_device
    x = _custom(64, 32, 500, 5)
    H, W, idx, tl, _ = to_device(x)
    with pytest.raises(ValueError):
        ckl.forward(H, W, idx, tl, torch.ones(64, dtype=torch.uint8))          # mask on the host
    with pytest.raises(ValueError):
        ckl.forward(H.cpu(), W, idx, tl)
    loss, lse, _ = ckl.forward(H, W, idx, tl)
    with pytest.raises(ValueError):
        ckl.backward(H, W, idx, tl, None, lse.cpu())                             # lse on the host
    with pytest.raises(ValueError):
        ckl.backward(H, W, idx, tl, None, lse[:10])                              # lse of another size
    with pytest.raises(ValueError):
        ckl.backward(H, W, idx, tl, None, lse.double())


def test_autograd_function():
    import torch

    import chunked_kl_loss_amd as ckl
    from tests.gpu_harness import to_device
    x = inputs(1, T=512)
    H, W, idx, tl, m = to_device(x)
    H.requires_grad_(True)
    W.requires_grad_(True)
    loss = ckl.chunked_kl_loss(H, W, idx, tl, m, chunk=256)
    (2.0 * loss).backward()
    ref = oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, grad_loss=2.0)
    assert abs(loss.item() - ref["loss"]) <= 2e-3 * ref["loss"]
    assert H.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    assert max_rel(H.grad.double().cpu().numpy(), ref["dH"]) <= 1e-2
    assert max_rel(W.grad.double().cpu().numpy(), ref["dW"]) <= 1e-2


def test_autograd_converts_layouts_and_index_types():
    # a strided view of H, int64 indices and bf16 teacher values give the
    # result of the contiguous int32 / fp32 call, and the gradient reaches
    # the tensor the view was taken from
    import torch

    import chunked_kl_loss_amd as ckl
    from tests.gpu_harness import to_device
    x = _custom(300, 64, 5000, 20)
    H, W, idx, tl, _ = to_device(x)
    tl = tl.to(torch.bfloat16).float()  # values that bf16 holds exactly
    for fused in (False, True):
        ref_H = H.clone().requires_grad_(True)
        ref = ckl.chunked_kl_loss(ref_H, W, idx, tl, chunk=128, fused=fused)
        ref.backward()
        wide = torch.zeros(x.T, 2 * x.d, dtype=H.dtype, device=H.device)
        wide[:, ::2] = H
        wide.requires_grad_(True)
        got = ckl.chunked_kl_loss(wide[:, ::2], W, idx.long(), tl.to(torch.bfloat16), chunk=128, fused=fused)
        got.backward()
        assert got.item() == ref.item()
        assert torch.equal(wide.grad[:, ::2], ref_H.grad)
        assert not wide.grad[:, 1::2].any()
    # batch dimensions: [2, 150, d] hidden states with a [2, 150] mask
    mask = torch.from_numpy((np.random.default_rng(3).random(x.T) < 0.7).astype(np.uint8)).to(H.device)
    for fused in (False, True):
        ref_H = H.clone().requires_grad_(True)
        ref = ckl.chunked_kl_loss(ref_H, W, idx, tl, mask, chunk=128, fused=fused)
        ref.backward()
        Hb = H.reshape(2, x.T // 2, x.d).clone().requires_grad_(True)
        got = ckl.chunked_kl_loss(Hb, W, idx.reshape(2, x.T // 2, -1), tl.reshape(2, x.T // 2, -1),
                                  mask.reshape(2, x.T // 2), chunk=128, fused=fused)
        got.backward()
        assert got.item() == ref.item()
        assert torch.equal(Hb.grad.reshape(x.T, x.d), ref_H.grad)


# ------------------------------------------- teacher given as log-probs ----
def test_logprob_teacher_fp32_full():
    x = with_logprob_teacher(inputs(0), n_neg_inf=5)
    assert np.exp(x.tlogit.astype(np.float64)).sum(axis=1).max() < 0.99
    say(f"case log-prob teacher fp32 T={x.T} V={x.V} K={x.K}")
    got = run_gpu(x, teacher_form=1, grad_loss=0.6)
    check_full(x, got, oracle_full(x, grad_loss=0.6, teacher_form=1), TOL["f32"], 1e-5)


def test_logprob_teacher_bf16_large_vocab():
    x = with_logprob_teacher(inputs(4, T=677))
    say(f"case log-prob teacher cfg4 slice T={x.T} masked={x.mask is not None}")
    got = run_gpu(x, teacher_form=1, chunk=300)
    check_full(x, got, oracle_full(x, teacher_form=1), TOL["bf16"], 2e-3)


def test_clustered_teacher_indices():
    # each row's K teacher indices are one run of consecutive vocabulary rows
    # (wrapping at V): a logit tile holds many of a token's indices at once,
    # so the gather walks several entries per tile, across tile boundaries
    x = _custom(300, 64, 5000, 100)
    rng = np.random.default_rng(11)
    start = rng.integers(0, x.V, size=x.T)
    idx = ((start[:, None] + np.arange(x.K)[None, :]) % x.V).astype(np.int32)
    x = dataclasses.replace(x, idx=idx)
    say(f"case clustered teacher indices T={x.T} V={x.V} K={x.K}")
    got = run_gpu(x, chunk=64, grad_loss=0.5)
    check_full(x, got, oracle_full(x, grad_loss=0.5), TOL["bf16"], 2e-3)
