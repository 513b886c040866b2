"""GPU parity of the one-call forward + backward (ckl_forward_backward: each
row chunk's logits are multiplied once and kept as exp(z - m) in the
workspace instead of being recomputed) against the fp64 oracle, element by
element, on the problems of the two-call tests: the tiny fp32 workload, the
4K x 32K bf16 workload, ragged reduced-row slices of the 201,088-vocabulary
workloads (one with packed-document masks), chunk sizes that give one or
many row chunks with a ragged last one, edge shapes and masks.

Tolerances as for the two-call path (bf16 inputs: loss 2e-3 relative, dH / dW
max-abs 1e-2 of max|ref|; fp32 inputs: 1e-5), which the extra rounding of
exp(z - m) to bf16 (one bf16 ulp, 2^-8 relative at most, on each non-teacher
entry of G before it is rescaled) stays well inside.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import make_inputs
from tests.gpu_harness import TOL, max_rel, run_gpu, run_gpu_fused, say
from tests.test_parity_gpu import _custom, check_full, oracle_full, with_logprob_teacher

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(cfg, seed=0, T=None):
    key = (cfg, seed, T)
    if key not in _cache:
        _cache[key] = make_inputs(cfg, seed=seed, T=T)
    return _cache[key]


def test_fused_tiny_fp32_full():
    x = inputs(0)
    say(f"case fused tiny fp32 T={x.T} d={x.d} V={x.V} K={x.K} chunk={x.chunk}")
    got = run_gpu_fused(x)
    e = check_full(x, got, oracle_full(x), TOL["f32"], 1e-5)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e}")


def test_fused_small_bf16_full():
    x = inputs(1)
    say(f"case fused small bf16 T={x.T} d={x.d} V={x.V} K={x.K} chunk={x.chunk}")
    got = run_gpu_fused(x)
    e = check_full(x, got, oracle_full(x), TOL["bf16"], 2e-3)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e}")


@pytest.mark.parametrize("cfg,T", [(2, 1000), (3, 677), (4, 677)])
def test_fused_large_vocab_row_slices(cfg, T):
    x = inputs(cfg, T=T)
    say(f"case fused cfg{cfg} slice T={x.T} chunk={x.chunk} masked={x.mask is not None}")
    got = run_gpu_fused(x)
    e = check_full(x, got, oracle_full(x), TOL["bf16"], 2e-3)
    say(f"  dH rel {e[0]:.2e} dW rel {e[1]:.2e}")


@pytest.mark.parametrize("chunk", [1, 300, 513, 100000])
def test_fused_chunk_sizes(chunk):
    # 256-row chunks (1 -> 4 chunks, the last ragged), 512 and 768 rows, one chunk
    import chunked_kl_loss_amd as ckl
    x = inputs(1, T=1000)
    plan = ckl.fused_plan(ckl.make_problem(x.T, x.d, x.V, x.K, chunk))
    say(f"case fused chunk={chunk} T={x.T} plan={plan}")
    got = run_gpu_fused(x, chunk=chunk, grad_loss=0.75)
    check_full(x, got, oracle_full(x, grad_loss=0.75), TOL["bf16"], 2e-3)


@pytest.mark.parametrize("T,d,V,K,dtype", [
    (1, 8, 16, 1, "bf16"),
    (3, 8, 1000, 7, "f32"),
    (130, 24, 300, 300, "bf16"),
    (257, 136, 129, 5, "bf16"),
    (64, 4096, 4096, 64, "bf16"),
    (300, 40, 777, 13, "f32"),
    (40, 64, 5000, 4096, "bf16"),  # K at its maximum
    (300, 64, 9000, 2, "bf16"),    # a short teacher list ending early in a long vocabulary walk
    (17, 16384, 700, 5, "bf16"),   # 16K hidden size
])
def test_fused_edge_shapes(T, d, V, K, dtype):
    x = _custom(T, d, V, K, dtype)
    say(f"case fused edge T={T} d={d} V={V} K={K} {dtype}")
    got = run_gpu_fused(x, chunk=3, grad_loss=1.5)
    check_full(x, got, oracle_full(x, grad_loss=1.5), TOL[dtype], 2e-3 if dtype == "bf16" else 1e-5)


def test_fused_masks_all_and_one():
    x = _custom(200, 64, 700, 9)
    say("case fused all rows masked")
    got = run_gpu_fused(x, mask=np.zeros(200, np.uint8))
    assert got["loss"] == 0.0
    assert (got["dH"] == 0).all() and (got["dW"] == 0).all() and (got["lse"] == 0).all()
    say("case fused one kept row")
    m = np.zeros(200, np.uint8)
    m[137] = 1
    got = run_gpu_fused(x, mask=m, grad_loss=3.0)
    check_full(x, got, oracle_full(x, grad_loss=3.0, mask=m), TOL["bf16"], 2e-3)


def test_fused_large_logit_range():
    # logits spread over ~+-60: exp(z - m) spans the whole fp32 exponent range
    # within a row, where a fixed reference point would overflow or flush
    x = _custom(300, 64, 3000, 17, "f32", seed=9)
    x.W *= 40.0
    say("case fused wide logit range fp32")
    got = run_gpu_fused(x, chunk=1)
    check_full(x, got, oracle_full(x), dict(loss_rel=1e-5, grad_rel=1e-4), 1e-4)


def test_fused_output_dtypes_and_default_grad():
    import torch
    x = _custom(300, 96, 1500, 11)
    say("case fused bf16 dH and dW outputs, grad_loss NULL")
    got = run_gpu_fused(x, dh_dtype=torch.bfloat16, dw_dtype=torch.bfloat16, chunk=5, grad_loss=None)
    check_full(x, got, oracle_full(x), TOL["bf16"], 2e-3)


def test_fused_validate_reports_bad_indices():
    import chunked_kl_loss_amd as ckl
    x = _custom(50, 16, 200, 6)
    run_gpu_fused(x, validate=True)
    y = _custom(50, 16, 200, 6)
    y.idx[9, 4] = y.idx[9, 1]
    say("case fused validate repeat")
    with pytest.raises(ckl.CklError) as e:
        run_gpu_fused(y, validate=True)
    assert e.value.status == 4
    # unchecked, out-of-range and negative entries must not fault (they match
    # no column); the call completes
    y.idx[7, 2] = 200
    y.idx[3, 0] = -1
    say("case fused unchecked bad indices")
    run_gpu_fused(y, validate=False)


def test_fused_matches_two_call_path():
    # the same loss up to the order of the split merges; gradients up to the
    # extra bf16 rounding of exp(z - m)
    x = inputs(1, T=1500)
    say("case fused vs two-call")
    a = run_gpu_fused(x, chunk=700, grad_loss=0.5)
    b = run_gpu(x, chunk=700, grad_loss=0.5)
    assert abs(a["loss"] - b["loss"]) <= 1e-6 * abs(b["loss"])
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-5)
    np.testing.assert_allclose(a["row_loss"], b["row_loss"], rtol=1e-5, atol=1e-5)
    # dW fp32 out: G's extra rounding only; dH bf16 out: plus one bf16 ulp of
    # the largest entry (see the full-size test)
    assert max_rel(a["dH"], b["dH"]) <= 2.0 ** -8 + 2 * 2.0 ** -9
    assert max_rel(a["dW"], b["dW"]) <= 4e-3


def test_fused_bitwise_deterministic():
    x = inputs(1, T=1500)
    say("case fused determinism")
    a = run_gpu_fused(x, chunk=100)
    b = run_gpu_fused(x, chunk=100)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_loss", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


def test_fused_step_under_graph_capture():
    # the one-call forward + backward (caller's workspace) captured in a HIP
    # graph and replayed with new inputs copied into the captured buffers:
    # every replay equals the eager call bit for bit
    import ctypes

    import torch

    from chunked_kl_loss_amd import _binding as B
    from tests.gpu_harness import to_device
    lib = B.load_library()
    xs = []
    for s in (21, 22):   # packed documents of 64..511 rows, the first quarter of each masked
        rng = np.random.default_rng(s)
        mask = np.ones(2200, np.uint8)
        t = 0
        while t < 2200:
            n = int(rng.integers(64, 512))
            mask[t:t + n // 4] = 0
            t += n
        xs.append(dataclasses.replace(_custom(2200, 256, 30000, 100, seed=s), mask=mask))
    x0 = xs[0]
    T, d, V, K = x0.T, x0.d, x0.V, x0.K
    prob = B.make_problem(T, d, V, K, 512, B.CKL_BF16, B.CKL_F32, B.CKL_F32, compact_mask=True)
    H, W, idx, tl, m = to_device(x0)
    g = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    lse = torch.zeros(T, dtype=torch.float32, device="cuda")
    dH = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    dW = torch.zeros((V, d), dtype=torch.float32, device="cuda")
    ws = torch.full((B.workspace_size(prob, 2),), 0xFF, dtype=torch.uint8, device="cuda")

    def call():
        B.check(lib.ckl_forward_backward(ctypes.byref(prob), H.data_ptr(), W.data_ptr(), idx.data_ptr(),
                                         tl.data_ptr(), m.data_ptr(), g.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                                         None, dH.data_ptr(), dW.data_ptr(), ws.data_ptr(), ws.numel(),
                                         torch.cuda.current_stream().cuda_stream), lib)

    def load(x):
        for dst, src in zip((H, W, idx, tl, m), to_device(x)):
            dst.copy_(src)

    refs = []
    for x in xs:
        load(x)
        call()
        torch.cuda.synchronize()
        refs.append([t.cpu().numpy().copy() for t in (loss, lse, dH, dW)])
    say("case one-call step captured in a graph")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(2):
        for x, ref in zip(xs, refs):
            load(x)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for t, r in zip((loss, lse, dH, dW), ref):
                assert np.array_equal(t.cpu().numpy(), r), rep


def test_fused_autograd_function():
    import torch

    import chunked_kl_loss_amd as ckl
    from tests.gpu_harness import to_device
    x = inputs(1, T=512)
    H, W, idx, tl, m = to_device(x)
    H.requires_grad_(True)
    W.requires_grad_(True)
    loss = ckl.chunked_kl_loss(H, W, idx, tl, m, chunk=256, fused=True)
    (2.0 * loss).backward()
    ref = oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, grad_loss=2.0)
    assert abs(loss.item() - ref["loss"]) <= 2e-3 * ref["loss"]
    assert H.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    assert max_rel(H.grad.double().cpu().numpy(), ref["dH"]) <= 1e-2
    assert max_rel(W.grad.double().cpu().numpy(), ref["dW"]) <= 1e-2
    # one chunk per dW update: the same gradients up to the fp32 grouping of dW
    H2 = H.detach().clone().requires_grad_(True)
    W2 = W.detach().clone().requires_grad_(True)
    (2.0 * ckl.chunked_kl_loss(H2, W2, idx, tl, m, chunk=256, fused=True, dw_group_rows=256)).backward()
    assert torch.equal(H2.grad, H.grad)
    assert max_rel(W2.grad.double().cpu().numpy(), W.grad.double().cpu().numpy()) <= 2 ** -7


def test_fused_logprob_teacher():
    x = with_logprob_teacher(inputs(0), n_neg_inf=5)
    say(f"case fused log-prob teacher fp32 T={x.T}")
    got = run_gpu_fused(x, teacher_form=1, grad_loss=0.6)
    check_full(x, got, oracle_full(x, grad_loss=0.6, teacher_form=1), TOL["f32"], 1e-5)
    y = with_logprob_teacher(inputs(2, T=1000))
    say(f"case fused log-prob teacher cfg2 slice T={y.T}")
    got = run_gpu_fused(y, teacher_form=1)
    check_full(y, got, oracle_full(y, teacher_form=1), TOL["bf16"], 2e-3)


def test_fused_odd_chunk_count():
    # three 256-row chunks (the last ragged) in one dW group: the update's k
    # range ends inside the last chunk
    import chunked_kl_loss_amd as ckl
    x = inputs(1, T=700)
    plan = ckl.fused_plan(ckl.make_problem(x.T, x.d, x.V, x.K, 200))
    assert plan["chunks"] == 3
    say(f"case fused odd chunk count T={x.T} plan={plan}")
    got = run_gpu_fused(x, chunk=200, grad_loss=1.25)
    check_full(x, got, oracle_full(x, grad_loss=1.25), TOL["bf16"], 2e-3)


def test_fused_partial_last_dw_group():
    # eleven 256-row chunks: a full group of eight, then a group of three
    # whose last chunk holds 40 rows (the dW update reads G k-major over
    # 2 * 256 + 256 rows of the second group)
    import chunked_kl_loss_amd as ckl
    x = inputs(1, T=2600)
    plan = ckl.fused_plan(ckl.make_problem(x.T, x.d, x.V, x.K, 256))
    assert plan["chunks"] == 11 and plan["rows"] == 256
    say(f"case fused partial last dW group T={x.T} plan={plan}")
    got = run_gpu_fused(x, chunk=256, grad_loss=0.75)
    check_full(x, got, oracle_full(x, grad_loss=0.75), TOL["bf16"], 2e-3)


def test_fused_clustered_teacher_indices():
    # each row's K teacher indices are one run of consecutive vocabulary rows
    # (wrapping at V): a logit tile holds many of a token's indices at once,
    # so the gather walks several entries per tile, across tile boundaries
    x = _custom(300, 64, 5000, 100)
    rng = np.random.default_rng(11)
    start = rng.integers(0, x.V, size=x.T)
    idx = ((start[:, None] + np.arange(x.K)[None, :]) % x.V).astype(np.int32)
    x = dataclasses.replace(x, idx=idx)
    say(f"case clustered teacher indices T={x.T} V={x.V} K={x.K}")
    got = run_gpu_fused(x, chunk=64, grad_loss=0.5)
    check_full(x, got, oracle_full(x, grad_loss=0.5), TOL["bf16"], 2e-3)
