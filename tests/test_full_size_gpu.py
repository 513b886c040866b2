"""GPU parity at full size (T up to 262,144 rows, V = 201,088, d = 2,880), in
the launch configuration the benchmark times, for both call paths.

At these sizes the fp64 oracle cannot evaluate everything, so the checks are
(the README page's CPU equivalence tests compare losses and gradients with the
dense reference; here that comparison is made on samples and closed forms):
  * >= 256 stratified rows computed one by one by the oracle (log-sum-exp,
    per-row KL, rows of dH): first/last rows, both sides of tile, forward
    chunk and backward G-block boundaries (in the packed kept-row order as
    well, for masked workloads), document starts, the last masked row before
    each kept span, and random rows;
  * >= 64 rows of dW from the oracle: vocabulary tile edges, the first and
    last rows, rows the teacher indices hit, random rows.  A dW row needs the
    log-sum-exp of every token row; the oracle takes the GPU's, after the
    sampled rows have checked it (at the 32K-row workload the oracle also
    computes every row's log-sum-exp itself);
  * properties that hold at any size: the loss is the masked mean of the row
    losses, masked rows give exact zeros, every column of dW sums to ~0
    (each row of the logit gradient sums to 0), results are bitwise
    reproducible;
  * a closed form over the whole problem: with every vocabulary row of W
    equal to c the student distribution is uniform, so LSE_t = h_t . c + ln V
    and dW[v] = sum_t s_t (1/V - p_t[v]) h_t -- also at 262,144 rows with the
    packed-document mask, where T x V = 5.3e10 exceeds 2^31.
Tolerances as in the element-wise tests (bf16 inputs: loss 2e-3 relative,
dH / dW 1e-2 of the largest reference magnitude, LSE 2e-3 absolute).
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs
from tests.gpu_harness import TOL, run_gpu, run_gpu_fused, say

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(cfg):
    if cfg not in _cache:
        _cache.clear()
        say(f"generating workload {cfg} ...")
        _cache[cfg] = make_inputs(cfg, seed=0)
    return _cache[cfg]


def _spread(values, k):
    """At most k of `values`, evenly spaced (all of them when there are few)."""
    values = list(values)
    if len(values) <= k:
        return values
    return [values[int(i)] for i in np.linspace(0, len(values) - 1, k)]


def sample_rows(x, chunk, n_total=256, seed=1):
    """>= n_total stratified token rows (see the module docstring)."""
    import chunked_kl_loss_amd as ckl
    prob = ckl.make_problem(x.T, x.d, x.V, x.K, chunk)
    fp, bp = ckl.fused_plan(prob), ckl.backward_plan(prob)
    T = x.T
    rows = {0, 1, 255, 256, T - 1, T - 2}
    cs, tc = fp["rows"], bp["Tc"]
    bounds = set(_spread(range(cs, T, cs), 24)) | set(_spread(range(tc, T, tc), 8)) | set(
        _spread(range(256, T, 256), 16))
    for b in bounds:
        rows.update({b - 1, b})
    if x.mask is not None:
        kept = np.nonzero(x.mask)[0]
        n = kept.size
        # the same boundaries in the packed order of the kept rows
        for b in set(_spread(range(cs, n, cs), 16)) | set(_spread(range(256, n, 256), 16)) | {n - 1}:
            rows.update({int(kept[b - 1]), int(kept[min(b, n - 1)])})
        starts = np.nonzero(np.diff(x.mask.astype(np.int8)) == 1)[0] + 1  # prompt span -> kept
        for s in _spread(starts, 12):
            rows.update({int(s), int(s) - 1})
    rng = np.random.default_rng(seed)
    while len(rows) < n_total:
        rows.add(int(rng.integers(0, T)))
    return np.array(sorted(r for r in rows if 0 <= r < T)), fp, bp


def sample_vocab_rows(x, n_total=64, seed=2):
    """>= n_total vocabulary rows of dW: tile edges, ends, teacher hits, random."""
    V = x.V
    v = {0, 1, 255, 256, 511, 512, V - 1, V - 2, (V // 256) * 256 - 1, (V // 256) * 256}
    v.update(int(i) for i in x.idx[:16, 0])            # the top teacher entry of some rows
    v.update(int(i) for i in x.idx[x.T // 2, :8])
    rng = np.random.default_rng(seed)
    while len(v) < n_total:
        v.add(int(rng.integers(0, V)))
    return np.array(sorted(i for i in v if 0 <= i < V))


def check_rows(x, got, rows, grad_loss=1.0):
    tol = TOL["bf16"]
    ref = oracle.kl_rows(x.H, x.W, x.idx, x.tlogit, rows, mask=x.mask, grad_loss=grad_loss)
    keep = np.ones(rows.size, bool) if x.mask is None else x.mask[rows] != 0
    np.testing.assert_allclose(got["lse"][rows][keep], ref["lse"][keep], rtol=0, atol=2e-3)
    np.testing.assert_allclose(got["row_loss"][rows][keep], ref["row_loss"][keep], rtol=tol["loss_rel"],
                               atol=tol["loss_rel"] * np.abs(ref["row_loss"][keep]).mean())
    scale = np.abs(ref["dH"][keep]).max()
    err = np.abs(got["dH"][rows][keep] - ref["dH"][keep]).max()
    assert err <= tol["grad_rel"] * scale, (err, scale)
    if (~keep).any():
        assert (got["dH"][rows][~keep] == 0).all()
        assert (got["lse"][rows][~keep] == 0).all() and (got["row_loss"][rows][~keep] == 0).all()
    return err / scale


def check_dw_rows(x, got, vrows, grad_loss=1.0, lse=None):
    """Oracle rows of dW given every row's log-sum-exp (the GPU's by default)."""
    lse = got["lse"] if lse is None else lse
    ref = oracle.dw_rows(x.H, x.W, x.idx, x.tlogit, vrows, lse, mask=x.mask, grad_loss=grad_loss)
    err = np.abs(got["dW"][vrows] - ref).max() / np.abs(ref).max()
    assert err <= TOL["bf16"]["grad_rel"], err
    return err


def check_properties(x, got):
    keep = np.ones(x.T, bool) if x.mask is None else x.mask != 0
    N = int(keep.sum())
    mean_rows = got["row_loss"][keep].sum() / N
    assert abs(got["loss"] - mean_rows) <= 1e-5 * abs(mean_rows)
    assert (got["dH"][~keep] == 0).all()
    assert (got["lse"][~keep] == 0).all()
    assert np.isfinite(got["dH"]).all() and np.isfinite(got["dW"]).all()
    colsum = got["dW"].sum(axis=0, dtype=np.float64)
    colabs = np.abs(got["dW"]).sum(axis=0, dtype=np.float64)
    assert (np.abs(colsum) <= 2e-3 * colabs).all(), np.max(np.abs(colsum) / colabs)


def full_check(x, got, chunk, label, dw=True):
    rows, fp, bp = sample_rows(x, chunk)
    e = check_rows(x, got, rows)
    msg = f"  {label}: {rows.size} sampled rows, dH rel err {e:.2e}"
    if dw:
        vrows = sample_vocab_rows(x)
        ew = check_dw_rows(x, got, vrows)
        msg += f"; {vrows.size} dW rows rel err {ew:.2e}"
    check_properties(x, got)
    say(msg + f"; loss {got['loss']:.6f}")


# ---------------------------------------------------------- closed form --
def _equal_rows(x0, seed=3):
    """x0 with every vocabulary row of W replaced by one random bf16 row c."""
    from synth import bf16_bits_to_f32
    rng = np.random.default_rng(seed)
    cbits = (rng.integers(0, 1 << 16, x0.d, dtype=np.uint32) & 0x3FFF | 0x3C00).astype(np.uint16)
    cbits[rng.random(x0.d) < 0.5] |= 0x8000
    Wb = np.ascontiguousarray(np.tile(cbits, (x0.V, 1)))   # what the GPU reads
    # (the fp32 copy is never read here: a broadcast view stands in for it)
    x = dataclasses.replace(x0, W=np.broadcast_to(bf16_bits_to_f32(cbits), (x0.V, x0.d)), W_bits=Wb)
    return x, bf16_bits_to_f32(cbits).astype(np.float64)


_dw_ref = {}


def _closed_form_dw(cfg, x, keep, s):
    """dW[v] = s (sum_kept h_t / V - sum_kept P[t, v] h_t), fp64 (cached per workload)."""
    import scipy.sparse as sp
    if cfg not in _dw_ref:
        p = oracle.teacher_probs(x.tlogit)
        kr = np.nonzero(keep)[0]
        Hk = x.H[kr].astype(np.float64)
        Pm = sp.csr_matrix((p[kr].ravel(), x.idx[kr].ravel().astype(np.int64),
                            np.arange(0, kr.size * x.K + 1, x.K)), shape=(kr.size, x.V))
        unit = Hk.sum(axis=0) / x.V - np.asarray(Pm.T @ Hk)   # the dW of s = 1
        _dw_ref.clear()
        _dw_ref[cfg] = unit
    return s * _dw_ref[cfg]


def _closed_form(cfg, path, chunk):
    # every vocabulary row equal to c: q_t is uniform, so
    #   LSE_t = h_t . c + ln V,  l_t = sum p log p + ln V,
    #   dW[v] = sum_t s_t (1/V - P[t, v]) h_t,  dH = (sum_v G[t, v]) c ~ 0,
    # over the whole problem (every row, every vocabulary tile and split)
    x, c = _equal_rows(inputs(cfg))
    keep = np.ones(x.T, bool) if x.mask is None else x.mask != 0
    N = int(keep.sum())
    chunk = chunk or x.chunk
    say(f"case closed form (equal vocabulary rows) cfg{cfg} {path} T={x.T} kept={N} chunk={chunk}")
    run = run_gpu if path == "two-call" else run_gpu_fused
    got = run(x, chunk=chunk, grad_loss=0.5, as64=False)
    hc = x.H.astype(np.float64) @ c
    np.testing.assert_allclose(got["lse"][keep], hc[keep] + math.log(x.V), rtol=0, atol=2e-3)
    assert (got["lse"][~keep] == 0).all()
    p = oracle.teacher_probs(x.tlogit)
    ent = (p * np.log(p)).sum(axis=1)
    np.testing.assert_allclose(got["row_loss"][keep], ent[keep] + math.log(x.V), rtol=2e-3, atol=2e-3)
    s = 0.5 / N
    dW_ref = _closed_form_dw(cfg, x, keep, s)
    err = np.abs(got["dW"] - dW_ref).max() / np.abs(dW_ref).max()
    say(f"  closed-form dW rel err {err:.2e}")
    assert err <= TOL["bf16"]["grad_rel"]
    # dH is (sum_v G[t, v]) c: zero up to the bf16 rounding of G
    g_abs = s * 2.0  # sum_v |G[t, v]| <= s (M + sum p) = 2 s
    assert np.abs(got["dH"]).max() <= 1e-2 * g_abs * np.abs(c).max()
    assert (got["dH"][~keep] == 0).all()


# Tests are grouped by workload (inputs are generated once per workload):
# the 32K-row headline, then 131,072 rows, then the 262,144-row packed
# documents.

def _fused_vs_two_call(got, ref):
    assert abs(got["loss"] - ref["loss"]) <= 1e-6 * abs(ref["loss"])
    np.testing.assert_allclose(got["lse"], ref["lse"], rtol=0, atol=1e-5)
    # dW is fp32 out: the paths differ by G's extra rounding only (u rounded
    # to bf16 before rescaling, <= 2^-9 relative per entry).  dH is bf16 out:
    # add one bf16 ulp of the largest entry (2^-8 of max|dH|) for two sums
    # that round to neighbouring bf16 values.
    bound = {"dW": 4e-3, "dH": 2.0 ** -8 + 2 * 2.0 ** -9}
    for k in ("dH", "dW"):
        err = np.abs(got[k] - ref[k]).max() / np.abs(ref[k]).max()
        say(f"  one-call vs two-call {k}: {err:.2e}")
        assert err <= bound[k], (k, err)


# ------------------------------------------------------ 32,768 rows (headline) --
def test_headline_two_call():
    x = inputs(2)
    say(f"case two-call cfg2 full T={x.T} chunk={x.chunk}")
    got = run_gpu(x, as64=False)
    full_check(x, got, x.chunk, "two-call cfg2")
    # the oracle's own fp64 log-sum-exp of every row (the expensive part),
    # then dW rows from it rather than from the GPU's
    lse = oracle.lse_rows(x.H, x.W, block=512)
    np.testing.assert_allclose(got["lse"], lse, rtol=0, atol=2e-3)
    e = check_dw_rows(x, got, sample_vocab_rows(x, n_total=40, seed=7), lse=lse)
    say(f"  every LSE row within 2e-3 of the oracle's; dW rows (oracle LSE) rel err {e:.2e}")
    b = run_gpu(x, as64=False)
    assert got["loss"] == b["loss"]
    for k in ("lse", "row_loss", "dH", "dW"):
        assert np.array_equal(got[k], b[k]), k
    say("  bitwise reproducible")


def test_headline_one_call():
    x = inputs(2)
    say(f"case one-call cfg2 full T={x.T} chunk={x.chunk}")
    got = run_gpu_fused(x, as64=False)
    full_check(x, got, x.chunk, "one-call cfg2")
    _fused_vs_two_call(got, run_gpu(x, as64=False))


def test_headline_closed_form():
    _closed_form(2, "two-call", None)


# ----------------------------------------------------------- 131,072 rows --
def test_long_two_call():
    x = inputs(3)
    say(f"case two-call cfg3 full T={x.T} chunk={x.chunk}")
    full_check(x, run_gpu(x, as64=False), x.chunk, "two-call cfg3")


def test_long_one_call():
    x = inputs(3)
    say(f"case one-call cfg3 full T={x.T} chunk={x.chunk}")
    full_check(x, run_gpu_fused(x, as64=False), x.chunk, "one-call cfg3")


# ------------------------------------- 262,144 rows, packed documents --
def test_packed_documents_chunk_sweep():
    x = inputs(4)
    w = WORKLOADS[4]
    base = None
    for chunk in w.chunk_sweep:
        say(f"case two-call cfg4 full T={x.T} kept={int(x.mask.sum())} chunk={chunk}")
        got = run_gpu(x, chunk=chunk, as64=False)
        full_check(x, got, chunk, f"two-call cfg4 chunk {chunk}", dw=chunk in (512, 2048, 8192))
        if base is None:
            base = got
        else:
            # chunk only reorders fp32 sums: the backward's sums between G
            # blocks (dW is fp32 out; dH is bf16 out, where a reordered sum may
            # round one bf16 ulp = 2^-8 apart); the forward's per-row arithmetic
            # does not depend on the chunk
            assert got["loss"] == pytest.approx(base["loss"], rel=1e-6)
            assert np.abs(got["lse"] - base["lse"]).max() <= 1e-5 * np.abs(base["lse"]).max()
            scale = np.abs(base["dW"]).max()
            assert np.abs(got["dW"] - base["dW"]).max() <= 1e-3 * scale
            assert np.abs(got["dH"] - base["dH"]).max() <= TOL["bf16"]["grad_rel"] * np.abs(base["dH"]).max()
        del got


@pytest.mark.parametrize("chunk", [512, 2048, 8192])
def test_packed_documents_one_call(chunk):
    x = inputs(4)
    say(f"case one-call cfg4 full T={x.T} kept={int(x.mask.sum())} chunk={chunk}")
    got = run_gpu_fused(x, chunk=chunk, as64=False)
    full_check(x, got, chunk, f"one-call cfg4 chunk {chunk}", dw=chunk == 2048)
    del got


@pytest.mark.parametrize("path,chunk", [("two-call", 512), ("two-call", 8192), ("one-call", 2048)])
def test_packed_documents_closed_form(path, chunk):
    _closed_form(4, path, chunk)
