"""Plain fp64 reference of the forward-KL distillation loss against a sparse
top-K teacher, with its gradients with respect to the hidden states H and the
output-head weights W.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously correct,
and independent of the HIP library.

Sources (the pages this follows):
  [README] "Chunked KL loss, running Knowledge Distillation locally in less
           <6GB VRAM" (the benchmark README): its method list, where Full Dense
           KL builds a dense teacher, compares it with the student's dense
           log-softmax and serves as the correctness baseline; and its
           objective section, whose sparse form of the loss is
           L(p, z) = sum_{v in S} p_v log p_v - sum_{v in S} p_v z_v + M logsumexp(z).
  [POST]   the author's announcement post: the teacher keeps only its top-100
           logits per position; the loss equals the standard KL divergence.
  [ABS]    "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and
           a Fused Chunked KL Loss", abstract: cached teacher top-K logits,
           fused chunked KL loss.

What is computed is the Full Dense KL baseline of [README], step by step:
  1. teacher probabilities: softmax over the K cached logits of each row
     (temperature 1), zero outside the cached support S;
  2. the dense teacher: those probabilities scattered into a [rows, V] tensor;
  3. student log-probabilities: z = H W^T, log q = z - logsumexp(z) per row;
  4. per-row forward KL(p || q) = sum_v p log p - sum_v p log q (0 log 0 = 0);
  5. the loss: the mean of the per-row KL over rows whose mask is 1
     (N = number of such rows; N = 0 gives loss 0 and zero gradients);
  6. the gradients: with s_t = grad_loss * mask_t / N, the logit gradient is
     G[t, v] = s_t * (M_t q[t, v] - P[t, v]), where M_t = sum_v P[t, v]
     (the teacher mass of the README formula); dH = G W and dW = G^T H.

Teacher forms.  ``teacher_form = 0`` (the default): the cached entries are
logits, renormalised over the K entries (M = 1 up to rounding).
``teacher_form = 1``: the cached entries are the teacher's log-probabilities
over its full vocabulary, truncated to the top K and used as given, so
p = exp(entry) and the mass M = sum_k p_k may be below 1 -- the general case
the README formula carries M for.  Steps 2-6 are unchanged: the per-row value
is sum_v p log p - sum_v p log q over the support, which is the README sparse
form with that M.

Readings where the pages are silent or garbled (the formula's definition of M
and the closed-form gradient were lost from the README text):
  * M is the teacher mass on its support, forced by expanding KL(p || q)
    with log q = z - logsumexp(z); with renormalised top-K logits M = 1.
  * the cached entries are logits, renormalised over the K entries
    ([POST] says the teacher's top-100 logits are what is stored).
  * the reduction is a mean over unmasked rows: PyTorch's KL divergence with
    batch-mean reduction over the kept token rows, which [POST] names as the
    loss this one equals.
  * rows are processed in blocks of ``block`` rows only to bound memory; the
    result does not depend on it beyond rounding (a pinned property).

Every function works in float64 and takes float32 (or exactly widened bf16)
arrays as given.
"""
from __future__ import annotations

import numpy as np

_F64 = np.float64


def teacher_probs(tlogit: np.ndarray, teacher_form: int = 0) -> np.ndarray:
    """Step 1: the teacher probabilities p[t, k] (fp64).

    teacher_form 0: softmax over k of the cached teacher logits, following
    [POST] (top-100 logits are cached) and [README] (the loss is evaluated
    against cached top-K teacher probabilities).  teacher_form 1: the cached
    entries are log-probabilities; p = exp(entry), not renormalised (the
    teacher mass M of the [README] formula is then sum_k p_k).
    """
    a = np.asarray(tlogit, dtype=_F64)
    if teacher_form == 1:
        return np.exp(a)
    if teacher_form != 0:
        raise ValueError("teacher_form must be 0 (logits) or 1 (log-probabilities)")
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=1, keepdims=True)


def dense_teacher(idx: np.ndarray, p: np.ndarray, V: int) -> np.ndarray:
    """Step 2: scatter the top-K probabilities into a dense [rows, V] tensor
    ([README], Full Dense KL paragraph).  Indices must be distinct within a
    row."""
    rows = idx.shape[0]
    P = np.zeros((rows, V), dtype=_F64)
    P[np.arange(rows)[:, None], np.asarray(idx, dtype=np.int64)] = p
    return P


def _xlogx(P: np.ndarray) -> np.ndarray:
    out = np.zeros_like(P)
    nz = P > 0
    out[nz] = P[nz] * np.log(P[nz])
    return out


def _logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def row_scale(mask: np.ndarray | None, T: int, grad_loss: float = 1.0):
    """Step 5/6 helper: (keep[T] bool, N, s[T]) with s_t = grad_loss*mask_t/N."""
    keep = np.ones(T, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    N = int(keep.sum())
    s = np.zeros(T, dtype=_F64)
    if N > 0:
        s[keep] = float(grad_loss) / N
    return keep, N, s


def _block(H64, W64, idx_b, p_b, s_b, V, want_grads):
    """Steps 2-4 and 6 for one block of rows (dense, fp64)."""
    z = H64 @ W64.T                                   # step 3: student logits
    lse = _logsumexp_rows(z)
    logq = z - lse[:, None]
    P = dense_teacher(idx_b, p_b, V)                  # step 2
    row_loss = _xlogx(P).sum(axis=1) - (P * logq).sum(axis=1)   # step 4
    if not want_grads:
        return lse, row_loss, None
    M = P.sum(axis=1)
    G = s_b[:, None] * (M[:, None] * np.exp(logq) - P)          # step 6
    return lse, row_loss, G


def kl_dense(H, W, idx, tlogit, mask=None, grad_loss: float = 1.0, block: int = 256,
             want_grads: bool = True, teacher_form: int = 0):
    """Full Dense KL loss, per-row LSE / KL, dH and dW in fp64.

    Returns a dict with ``loss`` (float), ``lse`` [T], ``row_loss`` [T] (both
    computed for every row, masked or not), ``dH`` [T, d], ``dW`` [V, d] (None
    when ``want_grads`` is False), ``N`` and ``keep``.
    """
    H = np.asarray(H)
    W = np.asarray(W)
    T, d = H.shape
    V = W.shape[0]
    W64 = W.astype(_F64)
    p = teacher_probs(tlogit, teacher_form)
    keep, N, s = row_scale(mask, T, grad_loss)
    lse = np.empty(T, dtype=_F64)
    row_loss = np.empty(T, dtype=_F64)
    dH = np.zeros((T, d), dtype=_F64) if want_grads else None
    dW = np.zeros((V, d), dtype=_F64) if want_grads else None
    for b0 in range(0, T, max(1, int(block))):
        b1 = min(T, b0 + max(1, int(block)))
        H64 = H[b0:b1].astype(_F64)
        l, r, G = _block(H64, W64, idx[b0:b1], p[b0:b1], s[b0:b1], V, want_grads)
        lse[b0:b1] = l
        row_loss[b0:b1] = r
        if want_grads:
            dH[b0:b1] = G @ W64
            dW += G.T @ H64
    loss = float(row_loss[keep].sum() / N) if N > 0 else 0.0   # step 5
    return dict(loss=loss, lse=lse, row_loss=row_loss, dH=dH, dW=dW, N=N, keep=keep)


def kl_rows(H, W, idx, tlogit, rows, mask=None, grad_loss: float = 1.0, block: int = 64,
            teacher_form: int = 0):
    """The same quantities for selected rows only: lse, row_loss and dH rows.

    Each row's values depend on that row alone (plus N through the mask), so
    this is the dense definition restricted to ``rows``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    T = np.asarray(H).shape[0]
    V = np.asarray(W).shape[0]
    W64 = np.asarray(W).astype(_F64)
    _, N, s = row_scale(mask, T, grad_loss)
    p = teacher_probs(np.asarray(tlogit)[rows], teacher_form)
    out_lse = np.empty(rows.size, dtype=_F64)
    out_loss = np.empty(rows.size, dtype=_F64)
    out_dH = np.empty((rows.size, W64.shape[1]), dtype=_F64)
    for b0 in range(0, rows.size, block):
        sel = rows[b0:b0 + block]
        H64 = np.asarray(H)[sel].astype(_F64)
        l, r, G = _block(H64, W64, np.asarray(idx)[sel], p[b0:b0 + block], s[sel], V, True)
        out_lse[b0:b0 + sel.size] = l
        out_loss[b0:b0 + sel.size] = r
        out_dH[b0:b0 + sel.size] = G @ W64
    return dict(lse=out_lse, row_loss=out_loss, dH=out_dH, N=N)


def lse_rows(H, W, block: int = 256) -> np.ndarray:
    """logsumexp over the full vocabulary of z = H W^T for every row (fp64)."""
    H = np.asarray(H)
    W64 = np.asarray(W).astype(_F64)
    out = np.empty(H.shape[0], dtype=_F64)
    for b0 in range(0, H.shape[0], block):
        out[b0:b0 + block] = _logsumexp_rows(H[b0:b0 + block].astype(_F64) @ W64.T)
    return out


def dw_rows(H, W, idx, tlogit, vrows, lse, mask=None, grad_loss: float = 1.0,
            block: int = 4096, teacher_form: int = 0) -> np.ndarray:
    """Rows ``vrows`` of dW = G^T H, given the fp64 LSE of every row (from
    ``lse_rows``).  Column v of G only needs z[:, v] = H w_v and the teacher
    entries equal to v."""
    H = np.asarray(H)
    T = H.shape[0]
    vrows = np.asarray(vrows, dtype=np.int64)
    Wsel = np.asarray(W)[vrows].astype(_F64)          # [R, d]
    p = teacher_probs(tlogit, teacher_form)
    _, N, s = row_scale(mask, T, grad_loss)
    M = p.sum(axis=1)
    # teacher probability at (t, vrows[j]); zero when vrows[j] is not in S_t
    Psel = np.zeros((T, vrows.size), dtype=_F64)
    pos = {int(v): j for j, v in enumerate(vrows)}
    idx = np.asarray(idx)
    hit_t, hit_k = np.nonzero(np.isin(idx, vrows))
    for t, k in zip(hit_t, hit_k):
        Psel[t, pos[int(idx[t, k])]] = p[t, k]
    out = np.zeros((vrows.size, H.shape[1]), dtype=_F64)
    for b0 in range(0, T, block):
        H64 = H[b0:b0 + block].astype(_F64)
        z = H64 @ Wsel.T                                   # [B, R]
        q = np.exp(z - np.asarray(lse)[b0:b0 + block, None])
        G = s[b0:b0 + block, None] * (M[b0:b0 + block, None] * q - Psel[b0:b0 + block])
        out += G.T @ H64
    return out


def kl_sparse_loss(H, W, idx, tlogit, mask=None, block: int = 256, teacher_form: int = 0):
    """The README's sparse form of the same objective, evaluated separately:
    l_t = sum_k p log p - sum_k p z[t, idx_k] + M_t * logsumexp(z_t),
    with only the log-normaliser spanning the vocabulary.  Returns
    (loss, row_loss[T])."""
    H = np.asarray(H)
    W64 = np.asarray(W).astype(_F64)
    T = H.shape[0]
    p = teacher_probs(tlogit, teacher_form)
    keep, N, _ = row_scale(mask, T)
    row_loss = np.empty(T, dtype=_F64)
    idx = np.asarray(idx, dtype=np.int64)
    for b0 in range(0, T, block):
        H64 = H[b0:b0 + block].astype(_F64)
        z = H64 @ W64.T
        lse = _logsumexp_rows(z)
        pb = p[b0:b0 + block]
        zg = np.take_along_axis(z, idx[b0:b0 + block], axis=1)
        ent = (pb * np.log(np.where(pb > 0, pb, 1.0))).sum(axis=1)
        row_loss[b0:b0 + block] = ent - (pb * zg).sum(axis=1) + pb.sum(axis=1) * lse
    loss = float(row_loss[keep].sum() / N) if N > 0 else 0.0
    return loss, row_loss
