"""GPU parity on drawn problem shapes: both paths against the fp64 oracle.

Each seed draws a problem from the space the C ABI accepts -- row count,
hidden size (a multiple of 8), vocabulary size, teacher entries K <= V,
chunk, input dtype, an optional mask with or without row packing, the
teacher form (logits, or log-probabilities with mass below one) and the
incoming gradient -- and checks the two-call path (ckl_forward +
ckl_backward) and the one-call path (ckl_forward_backward) element by
element against the oracle, to the tolerances of the other parity tests
(bf16: loss 2e-3 relative, dH / dW 1e-2 of the largest reference entry, LSE
2e-3 absolute; fp32: 1e-5; bf16 gradient outputs: 1e-2).  A wider draw adds
larger problems, bf16 gradient outputs, the device index check and the
one-call path's dW-group budget; a third draws ragged vocabulary shards
(ckl_shard_forward, ckl_shard_combine, ckl_backward per shard); a fourth
draws problems of up to 12K rows and 70K vocabulary rows, large enough for
plans with several G blocks, dH split parts and dW groups.  The seed
lists are fixed, so a failure names a reproducible problem; every buffer the
binding allocates starts as NaN bytes (tests/conftest.py).
"""
import numpy as np
import pytest

from tests.gpu_harness import TOL, run_gpu, run_gpu_fused, say
from tests.test_parity_gpu import _custom, check_full, oracle_full, with_logprob_teacher

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    T = int(rng.integers(1, 700))
    d = 8 * int(rng.integers(1, 97))
    V = int(rng.integers(2, 6000))
    K = int(rng.integers(1, min(V, 300) + 1))
    chunk = int(rng.choice([1, 7, 64, 255, 256, 257, 1000, 4096]))
    mask = None
    if rng.random() < 0.5:
        mask = (rng.random(T) < rng.uniform(0.2, 0.95)).astype(np.uint8)
    compact = bool(rng.random() < 0.5)
    teacher_form = int(rng.random() < 0.25)
    grad_loss = float(rng.choice([1.0, 0.5, -2.0]))
    return dict(dtype=dtype, T=T, d=d, V=V, K=K, chunk=chunk, mask=mask, compact=compact,
                teacher_form=teacher_form, grad_loss=grad_loss)


@pytest.mark.parametrize("seed", range(24))
def test_drawn_problem(seed):
    c = draw(seed)
    x = _custom(c["T"], c["d"], c["V"], c["K"], c["dtype"], seed=seed)
    if c["teacher_form"]:
        x = with_logprob_teacher(x, seed=seed)
    kept = c["T"] if c["mask"] is None else int(c["mask"].sum())
    say(f"case drawn seed={seed} T={c['T']} d={c['d']} V={c['V']} K={c['K']} chunk={c['chunk']} "
        f"{c['dtype']} kept={kept} compact={c['compact']} teacher_form={c['teacher_form']} "
        f"grad_loss={c['grad_loss']}")
    ref = oracle_full(x, grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"])
    tol = TOL[c["dtype"]]
    lse_tol = 2e-3 if c["dtype"] == "bf16" else 1e-5
    args = dict(chunk=c["chunk"], grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"],
                compact=c["compact"])
    check_full(x, run_gpu(x, **args), ref, tol, lse_tol)
    check_full(x, run_gpu_fused(x, **args), ref, tol, lse_tol)


def draw_options(seed):
    """A wider draw: larger problems, output dtypes, the index check, the
    one-call path's dW-group budget."""
    rng = np.random.default_rng(5000 + seed)
    c = draw(seed + 100)
    c["T"] = int(rng.integers(1, 2000))
    c["d"] = 8 * int(rng.integers(1, 129))
    c["V"] = int(rng.integers(2, 20000))
    c["K"] = int(rng.integers(1, min(c["V"], 400) + 1))
    if c["mask"] is not None:
        c["mask"] = (rng.random(c["T"]) < rng.uniform(0.2, 0.95)).astype(np.uint8)
    c["dh_bf16"] = bool(rng.random() < 0.3)
    c["dw_bf16"] = bool(rng.random() < 0.3)
    c["validate"] = bool(rng.random() < 0.3)
    c["dw_group_rows"] = int(rng.choice([0, 1, 3 * max(c["chunk"], 1), 100000]))
    return c


@pytest.mark.parametrize("seed", range(32))
def test_drawn_problem_options(seed):
    import torch
    c = draw_options(seed)
    x = _custom(c["T"], c["d"], c["V"], c["K"], c["dtype"], seed=seed + 7)
    if c["teacher_form"]:
        x = with_logprob_teacher(x, seed=seed)
    kept = c["T"] if c["mask"] is None else int(c["mask"].sum())
    say(f"case drawn+ seed={seed} T={c['T']} d={c['d']} V={c['V']} K={c['K']} chunk={c['chunk']} "
        f"{c['dtype']} kept={kept} compact={c['compact']} teacher_form={c['teacher_form']} "
        f"grad_loss={c['grad_loss']} dH bf16={c['dh_bf16']} dW bf16={c['dw_bf16']} validate={c['validate']} "
        f"dw_group_rows={c['dw_group_rows']}")
    ref = oracle_full(x, grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"])
    tol = dict(TOL[c["dtype"]])
    if c["dh_bf16"] or c["dw_bf16"]:
        tol["grad_rel"] = TOL["bf16"]["grad_rel"]  # one bf16 rounding of the gradients
    lse_tol = 2e-3 if c["dtype"] == "bf16" else 1e-5
    args = dict(chunk=c["chunk"], grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"],
                compact=c["compact"], validate=c["validate"],
                dh_dtype=torch.bfloat16 if c["dh_bf16"] else torch.float32,
                dw_dtype=torch.bfloat16 if c["dw_bf16"] else torch.float32)
    check_full(x, run_gpu(x, **args), ref, tol, lse_tol)
    check_full(x, run_gpu_fused(x, dw_group_rows=c["dw_group_rows"], **args), ref, tol, lse_tol)


@pytest.mark.parametrize("seed", range(12))
def test_drawn_vocabulary_shards(seed):
    """Ragged vocabulary shards of a drawn problem, merged, against the oracle."""
    import dataclasses

    from tests.test_shards_gpu import check as check_shards
    from tests.test_shards_gpu import run_shards
    c = draw(seed + 200)
    rng = np.random.default_rng(7000 + seed)
    x = _custom(c["T"], c["d"], c["V"], c["K"], c["dtype"], seed=seed + 11)
    if c["teacher_form"]:
        x = with_logprob_teacher(x, seed=seed)
    x = dataclasses.replace(x, mask=c["mask"])
    n_shards = int(rng.integers(1, min(6, c["V"]) + 1))
    cuts = np.sort(rng.choice(np.arange(1, c["V"]), size=n_shards - 1, replace=False)) if n_shards > 1 else []
    bounds = [0] + [int(v) for v in cuts] + [c["V"]]
    say(f"case drawn shards seed={seed} T={c['T']} d={c['d']} V={c['V']} K={c['K']} {c['dtype']} "
        f"bounds={bounds} masked={c['mask'] is not None} teacher_form={c['teacher_form']}")
    ref = oracle_full(x, grad_loss=c["grad_loss"], teacher_form=c["teacher_form"])
    got = run_shards(x, bounds, grad_loss=c["grad_loss"], chunk=c["chunk"], teacher_form=c["teacher_form"])
    check_shards(x, got, ref, TOL[c["dtype"]], 2e-3 if c["dtype"] == "bf16" else 1e-5)


def draw_large(seed):
    """Problems large enough for multi-block plans: several G blocks in both
    directions, dH split parts, several dW groups, many vocabulary splits."""
    rng = np.random.default_rng(9000 + seed)
    T = int(rng.integers(2000, 12000))
    V = int(rng.integers(20000, 70000))
    mask = (rng.random(T) < rng.uniform(0.3, 0.95)).astype(np.uint8) if rng.random() < 0.5 else None
    return dict(dtype="f32" if rng.random() < 0.2 else "bf16", T=T, d=8 * int(rng.integers(8, 65)), V=V,
                K=int(rng.integers(1, 201)), chunk=int(rng.choice([256, 512, 1024, 2048, 4096])), mask=mask,
                compact=bool(rng.random() < 0.5), teacher_form=int(rng.random() < 0.25),
                grad_loss=float(rng.choice([1.0, 0.5, -2.0])))


@pytest.mark.parametrize("seed", range(6))
def test_drawn_large_problem(seed):
    c = draw_large(seed)
    x = _custom(c["T"], c["d"], c["V"], c["K"], c["dtype"], seed=seed + 13)
    if c["teacher_form"]:
        x = with_logprob_teacher(x, seed=seed)
    kept = c["T"] if c["mask"] is None else int(c["mask"].sum())
    say(f"case drawn large seed={seed} T={c['T']} d={c['d']} V={c['V']} K={c['K']} chunk={c['chunk']} "
        f"{c['dtype']} kept={kept} compact={c['compact']} teacher_form={c['teacher_form']} "
        f"grad_loss={c['grad_loss']}")
    ref = oracle_full(x, grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"])
    tol = TOL[c["dtype"]]
    lse_tol = 2e-3 if c["dtype"] == "bf16" else 1e-5
    args = dict(chunk=c["chunk"], grad_loss=c["grad_loss"], mask=c["mask"], teacher_form=c["teacher_form"],
                compact=c["compact"])
    check_full(x, run_gpu(x, **args), ref, tol, lse_tol)
    check_full(x, run_gpu_fused(x, **args), ref, tol, lse_tol)
