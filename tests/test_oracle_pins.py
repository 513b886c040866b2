"""Pins for the fp64 oracle: each test ties it to something other than itself
(hand-worked closed forms, finite differences, library routines it reduces to,
invariants of the KL divergence), chosen so that a dropped term, a wrong sign
or index, or a transposed operand in the oracle fails at least one of them.

All CPU; no GPU and no HIP library involved.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand_problem(rng, T, d, V, K, scale=1.0, masked=False):
    H = rng.standard_normal((T, d)) * scale
    W = rng.standard_normal((V, d)) / math.sqrt(d)
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    tl = rng.normal(0.0, math.sqrt(2.0), size=(T, K))
    mask = None
    if masked:
        mask = (rng.random(T) > 0.3).astype(np.uint8)
        mask[0] = 1
    return H, W, idx, tl, mask


# ---------------------------------------------------------------- golden ----
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    H = np.array(case["H"], dtype=np.float64)
    W = np.array(case["W"], dtype=np.float64)
    idx = np.array(case["idx"], dtype=np.int32)
    tl = np.array(case["tlogit"], dtype=np.float64)
    mask = None if case["mask"] is None else np.array(case["mask"], dtype=np.uint8)
    r = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=case["grad_loss"], block=1,
                        teacher_form=case.get("teacher_form", 0))
    assert r["loss"] == pytest.approx(case["loss"], rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(r["lse"], case["lse"], rtol=1e-13)
    for got, want in zip(r["row_loss"], case["row_loss"]):
        if want is not None:
            assert got == pytest.approx(want, rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(r["dH"], case["dH"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["dW"], case["dW"], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------ finite differences --
@pytest.mark.parametrize("masked", [False, True])
def test_gradients_match_central_differences(masked):
    rng = np.random.default_rng(11)
    T, d, V, K = 4, 8, 16, 4
    H, W, idx, tl, mask = _rand_problem(rng, T, d, V, K, masked=masked)
    g = 1.7
    r = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=g, block=3)
    h = 1e-6

    def f(Hx, Wx):
        return g * oracle.kl_dense(Hx, Wx, idx, tl, mask=mask, want_grads=False)["loss"]

    num_dH = np.zeros_like(H)
    for i in range(T):
        for j in range(d):
            Hp = H.copy(); Hp[i, j] += h
            Hm = H.copy(); Hm[i, j] -= h
            num_dH[i, j] = (f(Hp, W) - f(Hm, W)) / (2 * h)
    num_dW = np.zeros_like(W)
    for i in range(V):
        for j in range(d):
            Wp = W.copy(); Wp[i, j] += h
            Wm = W.copy(); Wm[i, j] -= h
            num_dW[i, j] = (f(H, Wp) - f(H, Wm)) / (2 * h)
    scale_h = np.abs(num_dH).max()
    scale_w = np.abs(num_dW).max()
    assert np.abs(r["dH"] - num_dH).max() <= 1e-7 * scale_h + 1e-12
    assert np.abs(r["dW"] - num_dW).max() <= 1e-7 * scale_w + 1e-12


# -------------------------------------------------------- KL invariants ----
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kl_nonnegative(seed):
    rng = np.random.default_rng(seed)
    H, W, idx, tl, _ = _rand_problem(rng, 32, 16, 64, 8, scale=3.0)
    r = oracle.kl_dense(H, W, idx, tl, want_grads=False)
    assert (r["row_loss"] >= -1e-12).all()
    assert r["loss"] > 0


def test_kl_zero_when_student_reproduces_teacher():
    # d = V, W = I: the student logits are H itself.  Put the teacher logits on
    # the support and a very negative value elsewhere: q equals the teacher
    # distribution to fp64 rounding, so KL and its gradient vanish.
    rng = np.random.default_rng(3)
    T, V, K = 6, 24, 5
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    tl = rng.normal(0, math.sqrt(2), size=(T, K))
    H = np.full((T, V), -1e4)
    H[np.arange(T)[:, None], idx] = tl
    r = oracle.kl_dense(H, np.eye(V), idx, tl)
    assert abs(r["loss"]) < 1e-13
    assert np.abs(r["row_loss"]).max() < 1e-13
    assert np.abs(r["dH"]).max() < 1e-15
    # shifting all student logits of a row by a constant changes nothing
    r2 = oracle.kl_dense(H + 7.25, np.eye(V), idx, tl)
    assert abs(r2["loss"]) < 1e-12


def test_logit_gradient_rows_sum_to_zero():
    # with W = I the hidden-state gradient is the logit gradient G itself
    rng = np.random.default_rng(4)
    T, V, K = 10, 20, 6
    H = rng.standard_normal((T, V)) * 2
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    tl = rng.normal(0, 1.4, size=(T, K))
    r = oracle.kl_dense(H, np.eye(V), idx, tl, grad_loss=3.0)
    np.testing.assert_allclose(r["dH"].sum(axis=1), 0.0, atol=1e-15)
    # and the gradient is not trivially zero
    assert np.abs(r["dH"]).max() > 1e-3


def test_block_size_invariance():
    rng = np.random.default_rng(5)
    H, W, idx, tl, mask = _rand_problem(rng, 23, 12, 40, 7, masked=True)
    ref = oracle.kl_dense(H, W, idx, tl, mask=mask, block=23)
    for B in (1, 7, 1000):
        r = oracle.kl_dense(H, W, idx, tl, mask=mask, block=B)
        assert r["loss"] == pytest.approx(ref["loss"], rel=1e-13)
        np.testing.assert_allclose(r["lse"], ref["lse"], rtol=1e-14)
        np.testing.assert_allclose(r["dH"], ref["dH"], rtol=1e-12, atol=1e-18)
        np.testing.assert_allclose(r["dW"], ref["dW"], rtol=1e-12, atol=1e-18)


def test_row_permutation():
    rng = np.random.default_rng(6)
    H, W, idx, tl, mask = _rand_problem(rng, 17, 8, 30, 5, masked=True)
    perm = rng.permutation(17)
    a = oracle.kl_dense(H, W, idx, tl, mask=mask)
    b = oracle.kl_dense(H[perm], W, idx[perm], tl[perm], mask=mask[perm])
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(b["dH"], a["dH"][perm], rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(b["dW"], a["dW"], rtol=1e-12, atol=1e-18)


# --------------------------------------------- reductions to library code --
def test_top1_teacher_equals_cross_entropy():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    T, d, V = 20, 6, 50
    H, W, idx, tl, _ = _rand_problem(rng, T, d, V, 1)
    r = oracle.kl_dense(H, W, idx, tl)
    z = torch.from_numpy(H) @ torch.from_numpy(W).T
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(idx[:, 0].astype(np.int64)))
    assert r["loss"] == pytest.approx(float(ce), rel=1e-13)


def test_full_support_equals_torch_kl_div_and_autograd():
    # K = V: the teacher is a full distribution; the loss must equal PyTorch's
    # KL divergence (sum / N) and its autograd gradients.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    T, d, V = 9, 5, 12
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d))
    idx = np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int32)
    tl = rng.normal(0, 2.0, size=(T, V))
    mask = np.array([1, 1, 0, 1, 1, 1, 0, 1, 1], dtype=np.uint8)
    r = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=0.5)

    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    target = torch.zeros(T, V, dtype=torch.float64)
    target.scatter_(1, torch.from_numpy(idx.astype(np.int64)), torch.softmax(torch.from_numpy(tl), dim=1))
    keep = torch.from_numpy(mask.astype(bool))
    logq = torch.log_softmax(Ht @ Wt.T, dim=1)
    kl = torch.nn.functional.kl_div(logq[keep], target[keep], reduction="sum") / int(keep.sum())
    (0.5 * kl).backward()
    assert r["loss"] == pytest.approx(float(kl.detach()), rel=1e-12)
    np.testing.assert_allclose(r["dH"], Ht.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_teacher_probs_closed_forms():
    tl = np.array([[0.0, 0.0], [math.log(3.0), 0.0], [2.0, -1.0]])
    p = oracle.teacher_probs(tl)
    np.testing.assert_allclose(p[0], [0.5, 0.5], rtol=1e-15)
    np.testing.assert_allclose(p[1], [0.75, 0.25], rtol=1e-15)
    sig = 1.0 / (1.0 + math.exp(-3.0))
    np.testing.assert_allclose(p[2], [sig, 1 - sig], rtol=1e-14)
    # shift invariance and normalisation on a large random case
    rng = np.random.default_rng(9)
    tl = rng.normal(0, 30, size=(50, 100))
    p = oracle.teacher_probs(tl)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.teacher_probs(tl + 123.0), p, rtol=1e-12)


# ---------------------------------------------------- sparse == dense ------
def test_sparse_formula_equals_dense():
    rng = np.random.default_rng(10)
    H, W, idx, tl, mask = _rand_problem(rng, 40, 16, 300, 12, scale=2.0, masked=True)
    dense = oracle.kl_dense(H, W, idx, tl, mask=mask, want_grads=False)
    loss, rows = oracle.kl_sparse_loss(H, W, idx, tl, mask=mask)
    assert loss == pytest.approx(dense["loss"], rel=1e-12)
    np.testing.assert_allclose(rows, dense["row_loss"], rtol=1e-11, atol=1e-13)


# ------------------------------------------------------ closed forms -------
def _entropy(p):
    scipy_stats = pytest.importorskip("scipy.stats")
    return scipy_stats.entropy(p, axis=1)


def test_zero_head_gives_log_v():
    rng = np.random.default_rng(12)
    T, d, V, K = 15, 8, 77, 9
    H, _, idx, tl, mask = _rand_problem(rng, T, d, V, K, masked=True)
    r = oracle.kl_dense(H, np.zeros((V, d)), idx, tl, mask=mask)
    np.testing.assert_allclose(r["lse"], math.log(V), rtol=1e-15)
    p = oracle.teacher_probs(tl)
    # KL(p || uniform) = log V - entropy(p)
    np.testing.assert_allclose(r["row_loss"], math.log(V) - _entropy(p), rtol=1e-12)


def test_equal_rows_head_closed_form():
    # every vocabulary row equal to c: z_t = (h_t . c) 1, q uniform;
    # LSE = h.c + log V, dH = 0 and dW[v] = sum_t s_t (1/V - P[t, v]) h_t.
    rng = np.random.default_rng(13)
    T, d, V, K = 14, 6, 40, 5
    H, _, idx, tl, mask = _rand_problem(rng, T, d, V, K, masked=True)
    c = rng.standard_normal(d)
    W = np.tile(c, (V, 1))
    g = 1.3
    r = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=g)
    np.testing.assert_allclose(r["lse"], H @ c + math.log(V), rtol=1e-14)
    assert np.abs(r["dH"]).max() < 1e-14
    p = oracle.teacher_probs(tl)
    keep = mask.astype(bool)
    N = keep.sum()
    want = np.zeros((V, d))
    for t in range(T):
        if not keep[t]:
            continue
        col = np.full(V, 1.0 / V)
        col[idx[t]] -= p[t]
        want += (g / N) * np.outer(col, H[t])
    np.testing.assert_allclose(r["dW"], want, rtol=1e-11, atol=1e-15)


# ------------------------------------------------------------ masking ------
def test_masked_rows_drop_out():
    rng = np.random.default_rng(14)
    H, W, idx, tl, mask = _rand_problem(rng, 19, 7, 33, 4, masked=True)
    keep = mask.astype(bool)
    a = oracle.kl_dense(H, W, idx, tl, mask=mask)
    b = oracle.kl_dense(H[keep], W, idx[keep], tl[keep])
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-13)
    assert (a["dH"][~keep] == 0).all()
    np.testing.assert_allclose(a["dH"][keep], b["dH"], rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-18)


def test_all_masked_gives_zero():
    rng = np.random.default_rng(15)
    H, W, idx, tl, _ = _rand_problem(rng, 5, 4, 10, 3)
    r = oracle.kl_dense(H, W, idx, tl, mask=np.zeros(5, np.uint8))
    assert r["loss"] == 0.0 and r["N"] == 0
    assert (r["dH"] == 0).all() and (r["dW"] == 0).all()


# ------------------------------------------------ row / column helpers -----
def test_row_and_column_helpers_agree_with_full():
    rng = np.random.default_rng(16)
    H, W, idx, tl, mask = _rand_problem(rng, 30, 9, 45, 6, masked=True)
    full = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=0.7)
    rows = np.array([0, 3, 29, 11])
    rr = oracle.kl_rows(H, W, idx, tl, rows, mask=mask, grad_loss=0.7, block=3)
    np.testing.assert_allclose(rr["lse"], full["lse"][rows], rtol=1e-14)
    np.testing.assert_allclose(rr["row_loss"], full["row_loss"][rows], rtol=1e-13)
    np.testing.assert_allclose(rr["dH"], full["dH"][rows], rtol=1e-12, atol=1e-18)
    lse = oracle.lse_rows(H, W, block=7)
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-14)
    vrows = np.array([0, 44, int(idx[0, 0]), 17])
    dw = oracle.dw_rows(H, W, idx, tl, vrows, lse, mask=mask, grad_loss=0.7, block=8)
    np.testing.assert_allclose(dw, full["dW"][vrows], rtol=1e-11, atol=1e-17)


# ------------------------------------------------ synthetic generator ------
def test_generator_recipe():
    x = make_inputs(0, seed=0)
    w = WORKLOADS[0]
    assert x.H.shape == (w.T, w.d) and x.W.shape == (w.V, w.d)
    s = np.sort(x.idx, axis=1)
    assert (s[:, 1:] != s[:, :-1]).all() and s.min() >= 0 and s.max() < w.V
    assert (np.diff(x.tlogit, axis=1) <= 0).all()
    y = make_inputs(0, seed=0)
    assert (x.H == y.H).all() and (x.idx == y.idx).all()
    b = make_inputs(1, seed=0, T=64)
    assert b.H_bits.dtype == np.uint16
    # bf16 widening is exact: rounding the widened values again is the identity
    from synth import bf16_round_bits
    assert (bf16_round_bits(b.H) == b.H_bits).all()
    from synth import packed_document_mask
    m, starts = packed_document_mask(np.random.default_rng(0), 262144)
    assert 0.22 < 1 - m.mean() < 0.28
    for a, b in zip(starts[:-1], starts[1:]):   # whole documents
        L = int(b - a)
        assert 512 <= L <= 8192
        n0 = int(round(0.25 * L))
        assert (m[a:a + n0] == 0).all() and (m[a + n0:b] == 1).all()


# ------------------------------------- teacher form 1: log-probabilities ----
def _truncated_logprobs(rng, T, K, extra=50):
    """Top-K log-probabilities of a softmax over K + extra classes: mass < 1."""
    full = rng.normal(0.0, 2.0, size=(T, K + extra))
    full -= full.max(axis=1, keepdims=True)
    logp = full - np.log(np.exp(full).sum(axis=1, keepdims=True))
    return np.sort(logp, axis=1)[:, ::-1][:, :K].copy()


def test_logprob_form_reduces_to_logits_when_normalised():
    # log-probabilities that sum to one (scipy's log_softmax of the logits)
    # describe the same teacher as the logits themselves
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(21)
    H, W, idx, tl, mask = _rand_problem(rng, 20, 12, 90, 7, scale=1.5, masked=True)
    a = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=0.7)
    b = oracle.kl_dense(H, W, idx, special.log_softmax(tl, axis=1), mask=mask, grad_loss=0.7, teacher_form=1)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-12)
    np.testing.assert_allclose(b["row_loss"], a["row_loss"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(b["dH"], a["dH"], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(b["dW"], a["dW"], rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("alpha", [0.25, 0.9])
def test_truncated_mass_scaling_closed_form(alpha):
    # p = alpha * softmax(l): the row value is alpha * (l_1 + log alpha) where
    # l_1 is the value for the normalised teacher (the M * LSE term carries
    # alpha), and the logit gradient s (M q - p) scales by alpha
    rng = np.random.default_rng(22)
    H, W, idx, tl, mask = _rand_problem(rng, 16, 10, 70, 6, scale=1.2, masked=True)
    one = oracle.kl_dense(H, W, idx, tl, mask=mask, grad_loss=1.3)
    lp = np.log(alpha) + (tl - tl.max(axis=1, keepdims=True))
    lp -= np.log(np.exp(tl - tl.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True))
    r = oracle.kl_dense(H, W, idx, lp, mask=mask, grad_loss=1.3, teacher_form=1)
    np.testing.assert_allclose(r["row_loss"], alpha * (one["row_loss"] + math.log(alpha)), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["dH"], alpha * one["dH"], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(r["dW"], alpha * one["dW"], rtol=1e-10, atol=1e-15)


def test_logprob_form_gradients_match_central_differences():
    rng = np.random.default_rng(23)
    T, d, V, K = 4, 6, 14, 4
    H, W, idx, _, mask = _rand_problem(rng, T, d, V, K, masked=True)
    lp = _truncated_logprobs(rng, T, K)
    assert (np.exp(lp).sum(axis=1) < 0.999).all()   # a real mass deficit
    g = 0.9
    r = oracle.kl_dense(H, W, idx, lp, mask=mask, grad_loss=g, teacher_form=1)
    h = 1e-6

    def f(Hx, Wx):
        return g * oracle.kl_dense(Hx, Wx, idx, lp, mask=mask, want_grads=False, teacher_form=1)["loss"]

    num_dH = np.zeros_like(H)
    for i in range(T):
        for j in range(d):
            Hp = H.copy(); Hp[i, j] += h
            Hm = H.copy(); Hm[i, j] -= h
            num_dH[i, j] = (f(Hp, W) - f(Hm, W)) / (2 * h)
    num_dW = np.zeros_like(W)
    for i in range(V):
        for j in range(d):
            Wp = W.copy(); Wp[i, j] += h
            Wm = W.copy(); Wm[i, j] -= h
            num_dW[i, j] = (f(H, Wp) - f(H, Wm)) / (2 * h)
    assert np.abs(r["dH"] - num_dH).max() <= 1e-7 * np.abs(num_dH).max() + 1e-12
    assert np.abs(r["dW"] - num_dW).max() <= 1e-7 * np.abs(num_dW).max() + 1e-12


def test_logprob_form_sparse_equals_dense():
    rng = np.random.default_rng(24)
    H, W, idx, _, mask = _rand_problem(rng, 30, 16, 200, 10, scale=2.0, masked=True)
    lp = _truncated_logprobs(rng, 30, 10)
    dense = oracle.kl_dense(H, W, idx, lp, mask=mask, want_grads=False, teacher_form=1)
    loss, rows = oracle.kl_sparse_loss(H, W, idx, lp, mask=mask, teacher_form=1)
    assert loss == pytest.approx(dense["loss"], rel=1e-12)
    np.testing.assert_allclose(rows, dense["row_loss"], rtol=1e-11, atol=1e-13)
