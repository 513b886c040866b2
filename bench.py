#!/usr/bin/env python3
"""Benchmark of the fused chunked forward-KL loss (forward + backward) on one
MI355X.

One step = the loss and its gradients dH, dW over one batch of synthetic
inputs that are resident in HBM before timing starts, either as
ckl_forward + ckl_backward (--path recompute: the backward recomputes the
logits chunk by chunk) or as one ckl_forward_backward call (--path fused: each
row chunk's logits are multiplied once and kept).  Default workload:
T = 32,768 rows, d = 2,880, V = 201,088, K = 100 cached teacher entries,
chunk = 2,048, bf16 H and W (the pages' 32K-context, 201,088-token-vocabulary
case).

Prints ONE JSON line with tokens/s, TFLOP/s (8 T V d useful flops per step),
the fraction of the bf16 dense MFMA peak, peak HBM, a roofline entry for the
dominant kernel (timed live with HIP events on the launch stream) and the fp64
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload 2] [--path fused|recompute]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
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


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


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
            "sample": f"first {rows} of {x.T} rows of the same workload (full d={x.d}, V={x.V}, K={x.K}); "
                      f"fp64 dense forward + backward in {dt:.1f} s",
            "seconds": dt}


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 1 GiB device-to-device copy (for scaling HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the loss shards by rows; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_kl_loss_amd as ckl
    from chunked_kl_loss_amd import _binding as B
    from synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
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
    H, W, idx, tl, mask = upload(x, dev)
    T, d, V, K = x.T, x.d, x.V, x.K
    in_code = B.CKL_BF16 if x.dtype == "bf16" else B.CKL_F32
    prob = B.make_problem(T, d, V, K, chunk, in_code, in_code, B.CKL_F32)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = ctypes.byref(prob)
    mp = None if mask is None else mask.data_ptr()
    peak = PEAK_BF16_TFLOPS if x.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    def measure(path: str, steps: int, warmup: int) -> dict:
        """Time `steps` steps of one path (inputs already resident); per-kernel event timing included."""
        fused = path == "fused"
        plan = B.fused_plan(prob) if fused else B.backward_plan(prob)
        torch.cuda.reset_peak_memory_stats(dev)
        ws_f = torch.empty(B.workspace_size(prob, 2 if fused else 0), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(1 if fused else B.workspace_size(prob, 1), dtype=torch.uint8, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        dH = torch.empty((T, d), dtype=H.dtype, device=dev)
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)

        def fwd():
            B.check(lib.ckl_forward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                    loss.data_ptr(), lse.data_ptr(), None, ws_f.data_ptr(), ws_f.numel(), sp), lib)

        def bwd():
            B.check(lib.ckl_backward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                     lse.data_ptr(), None, dH.data_ptr(), dW.data_ptr(), ws_b.data_ptr(),
                                     ws_b.numel(), sp), lib)

        def both():
            B.check(lib.ckl_forward_backward(P, H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(), mp,
                                             None, loss.data_ptr(), lse.data_ptr(), None, dH.data_ptr(),
                                             dW.data_ptr(), ws_f.data_ptr(), ws_f.numel(), sp), lib)

        if fused:
            fwd, bwd = both, (lambda: None)
        log(f"warmup {warmup} steps; path {path}, plan {plan}")
        for _ in range(warmup):
            fwd()
            bwd()
        torch.cuda.synchronize(dev)
        if not np.isfinite(loss.item()):
            raise RuntimeError("non-finite loss")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        ckl.timing_enable(True)
        torch.cuda.synchronize(dev)
        t_start = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            fwd()
            ev[i][1].record(stream)
            bwd()
            ev[i][2].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t_start
        ckl.timing_enable(False)
        fwd_ms = [e0.elapsed_time(e1) for e0, e1, _ in ev]
        bwd_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev]
        step_ms = wall * 1e3 / steps
        peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
        log(f"timed {steps} steps, path {path}: {step_ms:.2f} ms/step")
        kt = ckl.timing_read()
        del ws_f, ws_b, dH, dW, loss, lse
        torch.cuda.empty_cache()
        return dict(path=path, plan=plan, step_ms=step_ms, peak_gib=peak_gib, kt=kt,
                    fwd_ms=None if fused else float(np.mean(fwd_ms)),
                    bwd_ms=None if fused else float(np.mean(bwd_ms)),
                    events_min_ms=float(np.min(np.add(fwd_ms, bwd_ms))))

    m = measure(args.path, args.steps, args.warmup)
    fused = args.path == "fused"
    step_ms, kt, plan = m["step_ms"], m["kt"], m["plan"]

    # ---- per-kernel timing and roofline of the dominant kernel
    flops_step = 8.0 * T * V * d
    performed_step = (6.0 if fused else 8.0) * T * V * d
    algo_flops = {"fwd_lse": 2.0 * T * V * d, "gemm_dhdw": 4.0 * T * V * d}
    if not fused:
        algo_flops["bwd_grad"] = 2.0 * T * V * d
    kernels = {k: {"total_ms_per_step": ms / args.steps, "launches_per_step": n / args.steps,
                   "avg_launch_ms": (ms / n if n else 0.0)} for k, (ms, n) in kt.items()}
    dom = max(algo_flops, key=lambda k: kt[k][0])
    dom_ms, dom_n = kt[dom]
    achieved = algo_flops[dom] * args.steps / (dom_ms * 1e-3) / 1e12
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
                "avg_launch_ms": dom_ms / dom_n, "launches_per_step": dom_n / args.steps,
                "algorithmic_flops_per_step": algo_flops[dom],
                "algorithmic_flops_per_launch": algo_flops[dom] / (dom_n / args.steps)}
    tokens_s = T / (step_ms * 1e-3)
    tflops = flops_step / (step_ms * 1e-3) / 1e12
    n_valid = int(T if x.mask is None else x.mask.sum())
    result = {
        "metric": "fused KL fwd+bwd tokens/s and TFLOP/s (% MFMA bf16 peak); peak HBM GiB",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generator: H~N(0,1), W~N(0,1/d), K distinct uniform teacher indices, "
                "teacher logits N(0,2) sorted)",
        "config": {"workload": w.name, "T": T, "d": d, "V": V, "K": K, "chunk": chunk,
                   "masked_rows": T - n_valid, "parallelism": "single GPU", "path": args.path,
                   "plan": plan},
        "tflops": tflops,
        "tflops_note": "8 T V d flops per step, the method's count (forward, recomputed logits, dH, dW)"
                       + ("; the fused path multiplies 6 T V d of them (no recompute)" if fused else ""),
        "tflops_multiplied": performed_step / (step_ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * performed_step / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "peak_hbm_gib": m["peak_gib"],
        "fwd_ms": m["fwd_ms"],
        "bwd_ms": m["bwd_ms"],
        "step_ms_events_min": m["events_min_ms"],
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.compare:
        other = "recompute" if fused else "fused"
        o = measure(other, args.steps, args.warmup)
        result["other_path"] = {"path": other, "ms_per_step": o["step_ms"], "tokens_per_s": T / (o["step_ms"] * 1e-3),
                                "peak_hbm_gib": o["peak_gib"], "fwd_ms": o["fwd_ms"], "bwd_ms": o["bwd_ms"],
                                "plan": o["plan"],
                                "kernels_ms_per_step": {k: ms / args.steps for k, (ms, n) in o["kt"].items() if n}}
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
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
