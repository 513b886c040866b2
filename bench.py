#!/usr/bin/env python3
"""Benchmark of the fused chunked forward-KL loss (forward + backward) on one
MI355X.

One step = the loss and its gradients dH, dW over one batch of synthetic
inputs that are resident in HBM before timing starts, either as one
ckl_forward_backward call (--path fused: each row chunk's logits are
multiplied once and kept) or as ckl_forward + ckl_backward (--path recompute:
the backward recomputes the logits chunk by chunk, the pages' Full Chunked KL).
Default workload: T = 32,768 rows, d = 2,880, V = 201,088, K = 100 cached
teacher entries, chunk = 2,048, bf16 H and W (the pages' 32K-context,
201,088-token-vocabulary case).

Prints ONE JSON line: tokens/s, TFLOP/s (8 N V d useful flops per step over
the N unmasked rows; also the flops the path actually multiplies), the
fraction of the bf16 dense MFMA peak, peak HBM, a sampled-oracle parity check
made before timing, a roofline entry for the dominant kernel (per-kernel HIP
events on the launch stream, taken in a separate pass after the timed steps)
and the fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload 2] [--path fused|recompute]
    python bench.py --matrix     # workloads 1-4 and the packed-document chunk sweep,
                                 # one child process per (workload, chunk); failures -> FAILED rows
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_F32_MFMA_TFLOPS = 157.3  # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("chunked_kl_loss_amd/csrc/ckl_kernels.hip", "chunked_kl_loss_amd/csrc/ckl_tile.hpp",
                  "chunked_kl_loss_amd/csrc/ckl_common.hpp", "chunked_kl_loss_amd/csrc/ckl_api.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "fused KL fwd+bwd tokens/s and TFLOP/s (% MFMA bf16 peak); peak HBM GiB"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def upload(x, dev):
    """Host inputs -> device tensors (bf16 bit patterns are reinterpreted)."""
    import numpy as np
    import torch
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        H = torch.from_numpy(x.H).to(dev)
        W = torch.from_numpy(x.W).to(dev)
    idx = torch.from_numpy(x.idx).to(dev)
    tl = torch.from_numpy(x.tlogit).to(dev)
    mask = None if x.mask is None else torch.from_numpy(x.mask).to(dev)
    return H, W, idx, tl, mask


def cpu_baseline(x, rows: int):
    """The fp64 oracle, as it stands, on the first `rows` rows of the workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    sl = slice(0, rows)
    mask = None if x.mask is None else x.mask[sl]
    t0 = time.perf_counter()
    r = oracle.kl_dense(x.H[sl], x.W, x.idx[sl], x.tlogit[sl], mask=mask, block=128)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["loss"])
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {rows} of {x.T} rows of the same workload (full d={x.d}, V={x.V}, K={x.K}); "
                      f"fp64 dense forward + backward in {dt:.1f} s",
            "seconds": dt}


# A microbenchmark of the dense bf16 MFMA rate the chip sustains: every wave
# of 8-wave workgroups issues v_mfma_f32_32x32x16_bf16 back to back from
# registers (no memory traffic), its operands either N(0,1)-like bf16 values
# that change from one instruction to the next (what a contraction of random
# data sees) or one constant.  The board's power limit lowers the clock with
# the operands' switching activity, so the first figure is the practical
# ceiling for this path's data and the published 2.5 PFLOP/s the second's
# limit.
MFMA_PEAK_SRC = r"""
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16; return x;
}
__device__ __forceinline__ __bf16 val(unsigned h) {
  return (__bf16)(1.7f * ((h & 0xffff) / 65536.f + (h >> 16) / 65536.f - 1.f));
}
template <int RAND>
__global__ __launch_bounds__(512) void mfma_peak(int iters, float* out) {
  bf16x8 a[8], b[4];
  const unsigned s = blockIdx.x * 512 + threadIdx.x;
  for (int i = 0; i < 8; ++i)
    for (int e = 0; e < 8; ++e) a[i][e] = RAND ? val(mix(s * 131u + i * 8 + e)) : (__bf16)0.5f;
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 8; ++e) b[i][e] = RAND ? val(mix(s * 977u + 4099u + i * 8 + e)) : (__bf16)0.25f;
  f32x16 c[8] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[(i * 4 + j) & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], c[(i * 4 + j) & 7], 0, 0, 0);
  float t = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int r = 0; r < 16; ++r) t += c[j][r];
  out[blockIdx.x * 512 + threadIdx.x] = t;
}
int main() {
  const int iters = 2000, blocks = 1024;
  float* out;
  if (hipMalloc(&out, (size_t)blocks * 512 * 4) != hipSuccess) return 1;
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  for (int rnd = 1; rnd >= 0; --rnd) {
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      (void)hipEventRecord(e0);
      if (rnd) hipLaunchKernelGGL(mfma_peak<1>, dim3(blocks), dim3(512), 0, 0, iters, out);
      else hipLaunchKernelGGL(mfma_peak<0>, dim3(blocks), dim3(512), 0, 0, iters, out);
      (void)hipEventRecord(e1);
      (void)hipEventSynchronize(e1);
      float ms;
      (void)hipEventElapsedTime(&ms, e0, e1);
      if (ms < best) best = ms;
    }
    printf("%s %.3f\n", rnd ? "random" : "constant", (double)blocks * 8 * 32 * 32768.0 * iters / best / 1e9);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
"""


def mfma_peak():
    """Measured bf16 MFMA rate (TFLOP/s) with random and constant operands, from
    the microbenchmark above built with hipcc for gfx950 and run as a child
    process; None if it cannot be built or run."""
    import shutil
    import tempfile
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if not hipcc:
        return None
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "mfma_peak.hip"), os.path.join(tmp, "mfma_peak")
        with open(src, "w") as f:
            f.write(MFMA_PEAK_SRC)
        r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature", "-Xclang",
                            "-packed-fp32-ops", src, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            log(f"mfma peak probe did not build: {r.stderr[-300:]}")
            return None
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            return None
        vals = dict(line.split() for line in r.stdout.strip().splitlines())
        return {"random_operands_tflops": float(vals["random"]), "constant_operands_tflops": float(vals["constant"]),
                "unit": "TFLOP/s",
                "note": "v_mfma_f32_32x32x16_bf16 back to back from registers, 8 waves per CU, no memory traffic"}


def parity_sample(x, got, n_rows: int = 6, n_vrows: int = 4, seed: int = 5):
    """Sampled-oracle parity of one step's outputs: rows of LSE, per-row KL
    and dH computed one by one by the fp64 oracle, rows of dW from the
    oracle given the GPU's LSE (checked first on the sampled rows), and the
    loss against the masked mean of the GPU's row losses.  Tolerances are the
    parity tests' (bf16: loss 2e-3 relative, gradients 1e-2 of the largest
    reference entry; fp32: 1e-5)."""
    import numpy as np

    import oracle
    tol = dict(loss=2e-3, grad=1e-2, lse=2e-3) if x.dtype == "bf16" else dict(loss=1e-5, grad=1e-5, lse=1e-5)
    rng = np.random.default_rng(seed)
    keep = np.ones(x.T, bool) if x.mask is None else x.mask != 0
    kept = np.nonzero(keep)[0]
    rows = np.unique(np.concatenate([[kept[0], kept[-1]], rng.choice(kept, size=max(0, n_rows - 2))]))
    t0 = time.perf_counter()
    ref = oracle.kl_rows(x.H, x.W, x.idx, x.tlogit, rows, mask=x.mask)
    e_lse = float(np.abs(got["lse"][rows] - ref["lse"]).max())
    e_rl = float((np.abs(got["row_loss"][rows] - ref["row_loss"]) / np.abs(ref["row_loss"])).max())
    e_dh = float(np.abs(got["dH"][rows] - ref["dH"]).max() / np.abs(ref["dH"]).max())
    vrows = np.unique(np.concatenate([[0, x.V - 1], rng.integers(0, x.V, size=max(0, n_vrows - 2))]))
    dw_ref = oracle.dw_rows(x.H, x.W, x.idx, x.tlogit, vrows, got["lse"].astype(np.float64), mask=x.mask)
    e_dw = float(np.abs(got["dW"][vrows] - dw_ref).max() / np.abs(dw_ref).max())
    mean_rows = float(got["row_loss"][keep].astype(np.float64).sum() / keep.sum())
    e_loss = abs(got["loss"] - mean_rows) / abs(mean_rows)
    ok = (e_lse <= tol["lse"] and e_rl <= tol["loss"] and e_dh <= tol["grad"] and e_dw <= tol["grad"]
          and e_loss <= 1e-5 and bool((got["dH"][~keep] == 0).all()))
    return {"pass": bool(ok), "rows": [int(r) for r in rows], "vocab_rows": [int(v) for v in vrows],
            "lse_abs_err": e_lse, "row_loss_rel_err": e_rl, "dH_rel_err": e_dh, "dW_rel_err": e_dw,
            "loss_vs_row_mean_rel": e_loss, "oracle_s": time.perf_counter() - t0}


def run(args) -> dict:
    """One workload, one path, in this process.  Returns the result row."""
    import numpy as np
    import torch

    import chunked_kl_loss_amd as ckl
    from chunked_kl_loss_amd import _binding as B
    from synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    lib = ckl.load_library()
    w = WORKLOADS[args.workload]
    chunk = args.chunk or w.chunk
    log(f"generating workload {w.name} (seed {args.seed}) ...")
    t0 = time.perf_counter()
    x = make_inputs(w, seed=args.seed)
    log(f"  inputs ready in {time.perf_counter() - t0:.1f} s")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.empty(1, device=dev)  # initialise the context before resetting the peak counter
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]  # device memory free before the inputs (hipMemGetInfo)
    H, W, idx, tl, mask = upload(x, dev)
    T, d, V, K = x.T, x.d, x.V, x.K
    n_kept = int(T if x.mask is None else x.mask.sum())
    packed = mask is not None and not args.no_compact
    in_code = B.CKL_BF16 if x.dtype == "bf16" else B.CKL_F32
    prob = B.make_problem(T, d, V, K, chunk, in_code, in_code, B.CKL_F32, compact_mask=packed,
                          dw_group_rows=args.dw_group_rows)
    stream = torch.cuda.current_stream(dev)

    def cur():  # the stream calls go to: the current one (a graph capture switches it)
        return torch.cuda.current_stream(dev).cuda_stream
    P = ctypes.byref(prob)
    mp = None if mask is None else mask.data_ptr()
    peak = PEAK_BF16_TFLOPS if x.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    rows_mult = n_kept if packed else T  # rows whose logits the path multiplies

    def measure(path: str, steps: int, warmup: int, check: bool) -> dict:
        fused = path == "fused"
        plan = B.fused_plan(prob) if fused else B.backward_plan(prob)
        torch.cuda.reset_peak_memory_stats(dev)
        ws_f = torch.empty(B.workspace_size(prob, 2 if fused else 0), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(1 if fused else B.workspace_size(prob, 1), dtype=torch.uint8, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        row_loss = torch.empty(T, dtype=torch.float32, device=dev)
        dH = torch.empty((T, d), dtype=H.dtype, device=dev)
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)
        rl = row_loss.data_ptr() if check else None

        def fwd():
            B.check(lib.ckl_forward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                    loss.data_ptr(), lse.data_ptr(), rl, ws_f.data_ptr(), ws_f.numel(), cur()), lib)

        def bwd():
            B.check(lib.ckl_backward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                     lse.data_ptr(), None, dH.data_ptr(), dW.data_ptr(), ws_b.data_ptr(),
                                     ws_b.numel(), cur()), lib)

        def both():
            B.check(lib.ckl_forward_backward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                             None, loss.data_ptr(), lse.data_ptr(), rl, dH.data_ptr(),
                                             dW.data_ptr(), ws_f.data_ptr(), ws_f.numel(), cur()), lib)

        if fused:
            fwd, bwd = both, (lambda: None)
        log(f"warmup {warmup} steps; path {path}, plan {plan}")
        for _ in range(max(warmup, 1 if check else 0)):
            fwd()
            bwd()
        torch.cuda.synchronize(dev)
        if not np.isfinite(loss.item()):
            raise RuntimeError("non-finite loss")
        parity = None
        if check:
            got = dict(loss=float(loss.item()), lse=lse.cpu().numpy(), row_loss=row_loss.cpu().numpy(),
                       dH=dH.float().cpu().numpy(), dW=dW.cpu().numpy())
            parity = parity_sample(x, got)
            log(f"parity (sampled oracle rows): {parity}")
            del got
            rl = None  # the timed steps do not write the row losses
            torch.cuda.synchronize(dev)
            # the parity check's copies are not part of a step's footprint
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats(dev)
            fwd()
            bwd()
            torch.cuda.synchronize(dev)
        run_f, run_b = fwd, bwd
        if args.graph:
            # the step captured in HIP graphs (forward and backward apart, so
            # that the events still split them), replayed in the timed loop
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                fwd()
                bwd()
            stream.wait_stream(side)
            torch.cuda.synchronize(dev)
            graphs = []
            for f in ((fwd,) if fused else (fwd, bwd)):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    f()
                graphs.append(gr)
            run_f = graphs[0].replay
            run_b = (lambda: None) if fused else graphs[1].replay
            run_f()
            run_b()
            torch.cuda.synchronize(dev)
        if args.min_time > 0:
            # short steps: enough of them to fill min_time seconds
            torch.cuda.synchronize(dev)
            t1 = time.perf_counter()
            run_f()
            run_b()
            torch.cuda.synchronize(dev)
            steps = max(steps, int(np.ceil(args.min_time / max(time.perf_counter() - t1, 1e-6))))
        # timed steps: no per-kernel events
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize(dev)
        t_start = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            run_f()
            ev[i][1].record(stream)
            run_b()
            ev[i][2].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t_start
        fwd_ms = [e0.elapsed_time(e1) for e0, e1, _ in ev]
        bwd_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev]
        step_ms = wall * 1e3 / steps
        peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
        # what the runtime reports in use (hipMemGetInfo): inputs, outputs, the
        # workspaces as torch's allocator holds them, the library's code and
        # its static device array, against the free memory before the inputs
        used_gib = (free0 - torch.cuda.mem_get_info(dev)[0]) / 2**30
        log(f"timed {steps} steps, path {path}: {step_ms:.2f} ms/step")
        # per-kernel pass: the same steps again with the library's events on
        kt = None
        if args.kernel_steps > 0:
            ckl.timing_enable(True)
            for _ in range(args.kernel_steps):
                fwd()
                bwd()
            torch.cuda.synchronize(dev)
            kt = ckl.timing_read()
            ckl.timing_enable(False)
        del ws_f, ws_b, dH, dW, loss, lse, row_loss
        torch.cuda.empty_cache()
        return dict(path=path, plan=plan, step_ms=step_ms, peak_gib=peak_gib, used_gib=used_gib, kt=kt,
                    parity=parity, steps=steps,
                    fwd_ms=None if fused else float(np.mean(fwd_ms)),
                    bwd_ms=None if fused else float(np.mean(bwd_ms)),
                    fwd_ms_min=None if fused else float(np.min(fwd_ms)),
                    bwd_ms_min=None if fused else float(np.min(bwd_ms)),
                    events_mean_ms=float(np.mean(np.add(fwd_ms, bwd_ms))),
                    events_min_ms=float(np.min(np.add(fwd_ms, bwd_ms))))

    m = measure(args.path, args.steps, args.warmup, check=args.parity)
    fused = args.path == "fused"
    step_ms, kt, plan = m["step_ms"], m["kt"], m["plan"]

    flops_useful = 8.0 * n_kept * V * d
    flops_mult = (6.0 if fused else 8.0) * rows_mult * V * d
    roofline = None
    kernels = None
    if kt is not None:
        ks = args.kernel_steps
        algo_flops = {"fwd_lse": 2.0 * rows_mult * V * d, "gemm_dhdw": 4.0 * rows_mult * V * d}
        if not fused:
            algo_flops["bwd_grad"] = 2.0 * rows_mult * V * d
        kernels = {k: {"total_ms_per_step": ms / ks, "launches_per_step": n / ks,
                       "avg_launch_ms": (ms / n if n else 0.0)} for k, (ms, n) in kt.items()}
        dom = max(algo_flops, key=lambda k: kt[k][0])
        dom_ms, dom_n = kt[dom]
        achieved = algo_flops[dom] * ks / (dom_ms * 1e-3) / 1e12
        traffic = None
        try:
            with open(TRAFFIC_FILE) as fh:
                tr = json.load(fh)
            for e in tr.get("entries", []):
                ent = e.get("kernels", {}).get(dom)
                if (ent and e.get("source_hash") == kernel_source_hash() and e.get("workload") == w.name
                        and e.get("path") == args.path and chunk == w.chunk):
                    traffic = ent["hbm_bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            pass
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": traffic,
                    "avg_launch_ms": dom_ms / dom_n, "launches_per_step": dom_n / ks,
                    "algorithmic_flops_per_step": algo_flops[dom],
                    "algorithmic_flops_per_launch": algo_flops[dom] / (dom_n / ks),
                    "timing": f"HIP events around each launch on the launch stream, {ks} steps after the timed ones"}
    result = {
        "metric": METRIC,
        "value": T / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generator: H~N(0,1), W~N(0,1/d), K distinct uniform teacher indices, "
                "teacher logits N(0,2) sorted" + ("; packed documents, first quarter of each masked)"
                                                  if x.mask is not None else ")"),
        "config": {"workload": w.name, "T": T, "d": d, "V": V, "K": K, "chunk": chunk,
                   "masked_rows": T - n_kept, "packed_rows": packed, "parallelism": "single GPU",
                   "path": args.path, "plan": plan, "graph": bool(args.graph)},
        "kept_tokens_per_s": n_kept / (step_ms * 1e-3),
        "tflops": flops_useful / (step_ms * 1e-3) / 1e12,
        "tflops_note": "8 N V d flops per step over the N unmasked rows, the method's count (forward, "
                       "recomputed logits, dH, dW); tflops_multiplied counts what the path multiplies: "
                       + ("6 x rows V d (no recompute)" if fused else "8 x rows V d")
                       + (", rows = kept rows (masked rows packed away)" if packed else ", rows = T"),
        "tflops_multiplied": flops_mult / (step_ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * flops_mult / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "peak_hbm_gib": m["peak_gib"],
        "hbm_in_use_gib_mem_get_info": m["used_gib"],
        "fwd_ms": m["fwd_ms"],
        "bwd_ms": m["bwd_ms"],
        "fwd_ms_min": m["fwd_ms_min"],
        "bwd_ms_min": m["bwd_ms_min"],
        "step_ms_events_mean": m["events_mean_ms"],
        "step_ms_events_min": m["events_min_ms"],
        "parity": m["parity"],
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.compare:
        other = "recompute" if fused else "fused"
        o = measure(other, args.steps, args.warmup, check=False)
        result["other_path"] = {"path": other, "ms_per_step": o["step_ms"], "tokens_per_s": T / (o["step_ms"] * 1e-3),
                                "peak_hbm_gib": o["peak_gib"], "hbm_in_use_gib_mem_get_info": o["used_gib"],
                                "fwd_ms": o["fwd_ms"], "bwd_ms": o["bwd_ms"],
                                "fwd_ms_min": o["fwd_ms_min"], "bwd_ms_min": o["bwd_ms_min"],
                                "step_ms_events_min": o["events_min_ms"],
                                "tflops_multiplied": (6.0 if other == "fused" else 8.0) * rows_mult * V * d
                                / (o["step_ms"] * 1e-3) / 1e12,
                                "plan": o["plan"],
                                "kernels_ms_per_step": ({k: ms / args.kernel_steps for k, (ms, n) in o["kt"].items()
                                                         if n} if o["kt"] else None)}
        result["other_path"]["pct_bf16_peak"] = 100.0 * result["other_path"]["tflops_multiplied"] / PEAK_BF16_TFLOPS
    del H, W, idx, tl, mask
    torch.cuda.empty_cache()
    if args.copy_calibration:
        # a plain copy kernel of known size: reads 1 GiB and writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        result["copy_calibration_bytes"] = 1 << 30
        del src, dst
    if args.cpu_rows > 0:
        log(f"oracle CPU baseline on {args.cpu_rows} rows ...")
        result["cpu_baseline"] = cpu_baseline(x, min(args.cpu_rows, x.T))
    return result


def matrix(args, cases=None) -> dict:
    """Workloads 1-4 and the packed-document chunk sweep (or the given
    (workload, chunk or None) cases), each (workload, chunk, path) in its own
    child process (started before this process touches the GPU); a child that
    fails or runs out of memory gives a FAILED row and the sweep goes on."""
    from synth import WORKLOADS
    if cases is None:
        cases = [(1, None), (2, None), (3, None)] + [(4, c) for c in WORKLOADS[4].chunk_sweep]
    rows = []
    for wl, chunk in cases:
        for path in ("fused", "recompute"):
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", str(wl), "--path", path,
                   "--steps", str(args.steps), "--warmup", str(args.warmup), "--no-compare",
                   "--cpu-rows", "0", "--kernel-steps", "0", "--min-time", str(args.min_time or 1.0)]
            if chunk:
                cmd += ["--chunk", str(chunk)]
            name = f"workload {wl} chunk {chunk or WORKLOADS[wl].chunk} path {path}"
            log(f"matrix: {name}")
            t0 = time.perf_counter()
            try:
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=args.case_timeout)
                line = r.stdout.strip().splitlines()[-1] if r.returncode == 0 and r.stdout.strip() else ""
                row = json.loads(line) if line else None
                err = None if row else (r.stderr.strip().splitlines() or ["no output"])[-1]
            except subprocess.TimeoutExpired:
                row, err = None, f"timed out after {args.case_timeout} s"
            if row is None:
                rows.append({"workload": WORKLOADS[wl].name, "chunk": chunk or WORKLOADS[wl].chunk, "path": path,
                             "status": "FAILED", "error": err})
                log(f"  FAILED: {err}")
                continue
            c = row["config"]
            rows.append({"workload": c["workload"], "chunk": c["chunk"], "path": path, "status": "ok",
                         "T": c["T"], "kept_rows": c["T"] - c["masked_rows"], "packed_rows": c["packed_rows"],
                         "ms_per_step": row["ms_per_step"], "tokens_per_s": row["value"],
                         "tflops_useful": row["tflops"], "tflops_multiplied": row["tflops_multiplied"],
                         "pct_bf16_peak": row["pct_bf16_peak"], "peak_hbm_gib": row["peak_hbm_gib"],
                         "hbm_in_use_gib_mem_get_info": row["hbm_in_use_gib_mem_get_info"],
                         "fwd_ms": row["fwd_ms"], "bwd_ms": row["bwd_ms"], "fwd_ms_min": row["fwd_ms_min"],
                         "bwd_ms_min": row["bwd_ms_min"], "step_ms_events_min": row["step_ms_events_min"],
                         "parity": row["parity"], "steps": row["steps"], "wall_s": time.perf_counter() - t0})
            log(f"  {row['ms_per_step']:.1f} ms/step, peak {row['peak_hbm_gib']:.2f} GiB, "
                f"parity {'pass' if row['parity'] and row['parity']['pass'] else 'FAIL'}")
    return {"metric": METRIC, "matrix": rows, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "isolation": "one child process per (workload, chunk, path)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, help="synthetic workload id (0-4); 2 is the headline")
    ap.add_argument("--chunk", type=int, default=None, help="override the workload's chunk")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows of the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--path", choices=("fused", "recompute"), default="fused",
                    help="one ckl_forward_backward call per step, or ckl_forward + ckl_backward")
    ap.add_argument("--compare", action=argparse.BooleanOptionalAction, default=True,
                    help="after the timed path, also time the other one (reported under other_path)")
    ap.add_argument("--parity", action=argparse.BooleanOptionalAction, default=True,
                    help="check sampled rows against the fp64 oracle before timing")
    ap.add_argument("--kernel-steps", type=int, default=3,
                    help="steps of the separate per-kernel timing pass (0 = skip; no roofline entry)")
    ap.add_argument("--no-compact", action="store_true", help="masked workloads: compute masked rows too")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of HIP graphs captured from them (torch.cuda.graph)")
    ap.add_argument("--dw-group-rows", type=int, default=0, help="one-call path: rows per dW update (0 = default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 1 GiB device-to-device copy (for scaling HBM counters)")
    ap.add_argument("--matrix", action="store_true", help="the workload matrix, one child process per case")
    ap.add_argument("--mfma-peak", action=argparse.BooleanOptionalAction, default=True,
                    help="measure the sustained bf16 MFMA rate with a microbenchmark (hipcc, child process)")
    ap.add_argument("--case-timeout", type=int, default=300, help="--matrix: seconds per case")
    ap.add_argument("--min-time", type=float, default=0.0,
                    help="time at least this many seconds of steps (more than --steps where steps are short; "
                         "0 = exactly --steps; --matrix cases default to 1)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the loss shards by rows; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    peak = mfma_peak() if args.mfma_peak and not args.matrix else None  # before this process touches the GPU
    result = matrix(args) if args.matrix else run(args)
    if peak is not None:
        result["measured_mfma_peak"] = peak
        if result.get("roofline"):
            result["roofline"]["frac_of_measured_random_peak"] = (
                result["roofline"]["achieved"] / peak["random_operands_tflops"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
