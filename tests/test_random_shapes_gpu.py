"""GPU parity on drawn problem shapes: both paths against the fp64 oracle.

Each seed draws a problem from the space the C ABI accepts -- row count,
hidden size (a multiple of 8), vocabulary size, teacher entries K <= V,
chunk, input dtype, an optional mask with or without row packing, the
teacher form (logits, or log-probabilities with mass below one) and the
incoming gradient -- and checks the two-call path (ckl_forward +
ckl_backward) and the one-call path (ckl_forward_backward) element by
element against the oracle, to the tolerances of the other parity tests
(bf16: loss 2e-3 relative, dH / dW 1e-2 of the largest reference entry, LSE
2e-3 absolute; fp32: 1e-5).  The list of seeds is fixed, so a failure names
a reproducible problem.
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
