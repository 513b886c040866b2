"""Seeded synthetic inputs for the chunked forward-KL loss.

This module only draws random numbers and lays them out; it holds none of the
loss arithmetic. Both the fp64 oracle (through the tests) and the HIP path
(through the tests and the benchmark) take their inputs from here, so that
every implementation sees bit-identical data.

The workloads stand in for the output-head-only toy benchmark described in
"Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
Chunked KL Loss" (paper abstract) and in the repository README page ("Chunked
KL loss, running Knowledge Distillation locally in less <6GB VRAM", usage and
options table): synthetic hidden states, output weights and sparse top-K
teacher targets, generated deterministically.

Recipe (per workload and seed):
  * ``SeedSequence(seed).spawn(5)`` gives PCG64 streams for H, W, idx,
    teacher logits and the mask, in that order.
  * ``H ~ N(0, 1)`` of shape [T, d]; ``W ~ N(0, 1) / sqrt(d)`` of shape [V, d]
    (float32 draws).  bf16 workloads round both to bf16 with
    round-to-nearest-even.
  * ``idx``: K distinct indices in [0, V) per row, drawn uniformly with
    replacement; rows holding a repeat are drawn again until none does.
  * teacher logits: ``N(0, 2)`` (standard deviation sqrt(2)), float32, sorted
    in descending order along each row and paired with ``idx`` in draw order.
  * mask (packed-document workload only): documents with lengths uniform in
    {512, ..., 8192} are packed until T rows are filled (the last one is cut).
    In each document the first round(0.25 * L) positions (a prompt-like span)
    are masked out (0); the rest are kept (1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "Inputs",
    "make_inputs",
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "packed_document_mask",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    V: int
    K: int
    chunk: int
    dtype: str  # "f32" or "bf16": the dtype of H and W
    masked: bool = False
    chunk_sweep: tuple = ()


# The five workloads.  Shapes follow the pages' 32K-context, 201,088-token
# vocabulary case and the 4K..256K toy-benchmark sweep with top-100 teachers.
WORKLOADS = {
    0: Workload("tiny-f32", T=256, d=128, V=2048, K=16, chunk=64, dtype="f32"),
    1: Workload("small-bf16", T=4096, d=2048, V=32000, K=100, chunk=1024, dtype="bf16"),
    2: Workload("t32k-v201k-bf16", T=32768, d=2880, V=201088, K=100, chunk=2048, dtype="bf16"),
    3: Workload("t128k-v201k-bf16", T=131072, d=2880, V=201088, K=100, chunk=4096, dtype="bf16"),
    4: Workload("t256k-v201k-packed-bf16", T=262144, d=2880, V=201088, K=100, chunk=2048,
                dtype="bf16", masked=True, chunk_sweep=(512, 1024, 2048, 4096, 8192)),
}


@dataclasses.dataclass
class Inputs:
    """Host copies of one problem.

    ``H`` and ``W`` are float32 arrays holding exactly the values the GPU sees
    (for bf16 workloads they are the bf16 values widened to float32, which is
    exact).  ``H_bits``/``W_bits`` hold the raw bf16 bit patterns (uint16) for
    bf16 workloads and are ``None`` for f32 ones.
    """
    T: int
    d: int
    V: int
    K: int
    chunk: int
    dtype: str
    H: np.ndarray
    W: np.ndarray
    idx: np.ndarray        # int32 [T, K]
    tlogit: np.ndarray     # float32 [T, K]
    mask: np.ndarray | None  # uint8 [T] (1 = keep) or None (all kept)
    H_bits: np.ndarray | None = None
    W_bits: np.ndarray | None = None


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _distinct_indices(rng: np.random.Generator, T: int, K: int, V: int) -> np.ndarray:
    if K > V:
        raise ValueError("K must not exceed V")
    idx = rng.integers(0, V, size=(T, K), dtype=np.int64)
    while True:
        s = np.sort(idx, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0] if K > 1 else np.zeros(0, np.int64)
        if bad.size == 0:
            break
        idx[bad] = rng.integers(0, V, size=(bad.size, K), dtype=np.int64)
    return idx.astype(np.int32)


def packed_document_mask(rng: np.random.Generator, T: int, lo: int = 512, hi: int = 8192,
                         masked_frac: float = 0.25):
    """Return (mask uint8[T], document start offsets)."""
    mask = np.ones(T, dtype=np.uint8)
    starts = []
    pos = 0
    while pos < T:
        L = int(rng.integers(lo, hi + 1))
        starts.append(pos)
        n_masked = int(round(masked_frac * L))
        mask[pos:min(T, pos + n_masked)] = 0
        pos += L
    return mask, np.asarray(starts, dtype=np.int64)


def make_inputs(w: Workload | int, seed: int = 0, T: int | None = None) -> Inputs:
    """Draw one problem.  ``T`` overrides the workload's row count (the other
    sizes and the recipe stay the same)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    T = w.T if T is None else int(T)
    s_H, s_W, s_idx, s_tl, s_mask = np.random.SeedSequence(seed).spawn(5)
    rH, rW, ridx, rtl, rmask = (np.random.Generator(np.random.PCG64(s)) for s in (s_H, s_W, s_idx, s_tl, s_mask))

    H = rH.standard_normal((T, w.d), dtype=np.float32)
    W = rW.standard_normal((w.V, w.d), dtype=np.float32)
    W /= np.float32(math.sqrt(w.d))
    idx = _distinct_indices(ridx, T, w.K, w.V)
    tl = rtl.normal(0.0, math.sqrt(2.0), size=(T, w.K)).astype(np.float32)
    tl = -np.sort(-tl, axis=1)
    mask = packed_document_mask(rmask, T)[0] if w.masked else None

    H_bits = W_bits = None
    if w.dtype == "bf16":
        H_bits = bf16_round_bits(H)
        W_bits = bf16_round_bits(W)
        H = bf16_bits_to_f32(H_bits)
        W = bf16_bits_to_f32(W_bits)
    elif w.dtype != "f32":
        raise ValueError(w.dtype)
    return Inputs(T=T, d=w.d, V=w.V, K=w.K, chunk=w.chunk, dtype=w.dtype, H=H, W=W,
                  idx=np.ascontiguousarray(idx), tlogit=np.ascontiguousarray(tl), mask=mask,
                  H_bits=H_bits, W_bits=W_bits)
