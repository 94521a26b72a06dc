#!/usr/bin/env python3
"""Benchmark of the verifier acceptance step (libspecverify) on one MI355X.

A step is one sv_verify call over one batch of synthetic logits already
resident in HBM: validation, the row-profile kernels (the HBM-streaming part),
the acceptance kernel and the additional-token sampler.

Prints ONE JSON line:
  value        verified positions per second, P = sum_b (m_b + 1) per step
  roofline     the row-profile kernels: algorithmic bytes per launch (each
               row a session's rule reads, once) / their average duration
               measured with hipEvents recorded on the launch stream, against
               the 8 TB/s HBM peak; traffic = counter-measured HBM bytes per
               launch when known for the current kernels (else null)
  cpu_baseline the oracle (plain single-threaded C, binary64) on this host,
               on a bounded sample of the same workload's sessions
Default workload: B=256, M=8, V=128256, bf16, T=0.7, top_k=50, top_p=0.9.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "verified positions/sec (B*(M+1)/s) + achieved HBM GB/s vs 8 TB/s peak"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "b256_topk_topp"

# Counter-measured HBM traffic per launch of the row kernels (bytes), keyed by
# (workload, kernel revision); filled from rocprofv3 FETCH_SIZE/WRITE_SIZE runs.
KERNEL_REVISION = "rows-generic-v1"
MEASURED_TRAFFIC = {}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, budget_s: float):
    """Time the oracle on the first sessions of the workload (bounded sample)."""
    import numpy as np

    import oracle
    from token_sampling_amd import workloads as W

    oracle.lib()
    n = 1
    done_sessions = 0
    positions = 0
    elapsed = 0.0
    while done_sessions < w.B and elapsed < budget_s:
        idx = list(range(done_sessions, min(w.B, done_sessions + n)))
        h = W.to_numpy(w, sessions=idx)
        t0 = time.perf_counter()
        oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"],
                      h["seed"], h["round"], diagnostics=False)
        dt = time.perf_counter() - t0
        elapsed += dt
        positions += int((np.asarray(h["m"], dtype=np.int64) + 1).sum())
        done_sessions += len(idx)
        per = dt / len(idx)
        n = max(1, min(64, int((budget_s - elapsed) / max(per, 1e-6) / 2)))
    return {
        "value": positions / elapsed,
        "unit": "positions/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"sessions 0..{done_sessions - 1} of {w.name} (P={positions}), "
                  f"{elapsed:.1f} s single-threaded",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--sessions", type=int, default=None,
                    help="diagnostic only: the workload's first N sessions instead of all")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the verifier step shards by session with no exchange, so N GPUs run N "
              "independent copies of this single-GPU step.", file=sys.stderr)
        sys.exit(2)

    import torch

    import token_sampling_amd as sv
    from token_sampling_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"[bench] building workload {args.workload}")
    w = W.make(args.workload, device="cuda", sessions=args.sessions)
    smp = w.sampling_tensor(dev)
    B, M, V = w.B, w.M, w.V
    P = w.positions()
    alg_bytes = w.algorithmic_bytes()
    ws = torch.empty(sv.workspace_bytes(B, M, V), dtype=torch.uint8, device=dev)
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty((B, M + 1), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, smp, w.seed, w.round,
                  workspace=ws, out=out, stream=stream, row_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    row_ev = [(sv.HipEvent(), sv.HipEvent()) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step(row_ev[k])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    rows_ms = [a.elapsed_ms(b) for a, b in row_ev]
    ms_per_step = total_ms / args.steps
    rows_avg_ms = sum(rows_ms) / len(rows_ms)
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step, row kernels {rows_avg_ms:.4f} ms")

    a = out["accepted_len"].cpu()
    achieved = alg_bytes / (rows_avg_ms * 1e-3) / 1e9
    traffic = MEASURED_TRAFFIC.get((args.workload, KERNEL_REVISION))
    result = {
        "metric": METRIC,
        "value": P / (ms_per_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "B": B, "M": M, "V": V,
            "logits": "bf16" if w.target.dtype == torch.bfloat16 else "fp32",
            "positions_per_step": P, "algorithmic_bytes_per_step": alg_bytes,
            "mean_accepted": float(a[a >= 0].float().mean()) if (a >= 0).any() else None,
            "bad_proposals": int((a == sv.S_BAD_PROPOSAL).sum()),
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "row-profile kernels", "ms_per_launch": rows_avg_ms,
        },
    }
    if args.cpu_budget > 0:
        log(f"[bench] oracle CPU baseline (~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
