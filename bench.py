#!/usr/bin/env python3
"""Benchmark of the verifier acceptance step (libspecverify) on one MI355X.

A step is one sv_verify call (sv_verify_sdcp with --sdcp, sv_verify_qrows with
--qrows, sv_verify_early with --early W) over one batch of synthetic logits
already resident in HBM: the single-pass row kernel (session checks and the row
profiles, the HBM-streaming part), the generic row kernel, and the per-session
kernel (acceptance and the additional token).  With --early the rows are read in
windows of positions, and the roofline line counts the rows the sessions need
(a+1 target rows and, for rule 2, a+1 draft rows) over the time of all the
windows' row and advance kernels.

Prints ONE JSON line:
  value        verified positions per second, P = sum_b (m_b + 1) per step
  roofline     the dominant row kernel: algorithmic bytes per launch (each
               row it handles, once) / its average duration measured with
               hipEvents recorded on the launch stream, against the 8 TB/s HBM
               peak; traffic = counter-measured HBM bytes per launch when known
               for the current kernel revision (else null)
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

# Counter-measured HBM traffic per launch of the dominant kernel (bytes), keyed
# by (workload, kernel, kernel revision); filled from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs and valid only for the revision they were taken on.
KERNEL_REVISION = "stream-v5"
MEASURED_TRAFFIC = {
    # FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, scaled by a 1 GiB copy kernel
    ("b256_topk_topp", "k_rows_stream", "stream-v2"): 1_119_476_736,
    ("b256_topk_topp", "k_rows_stream", "stream-v3"): 1_119_487_488,
    ("b256_topk_topp", "k_rows_stream", "stream-v4"): 1_119_499_072,
    ("b256_topk_topp", "k_rows_stream", "stream-v5"): 1_119_496_295,
    ("b64", "k_rows_split<4>", "stream-v5"): 38_273_434,
    ("ragged", "k_rows_stream", "stream-v5"): 2_450_512_384,
    ("large", "k_rows_stream", "stream-v5"): 34_218_138_829,
}
# VALU busy (rocprofv3 derived counter VALUBusy: VALU cycles over GPU-busy
# cycles per CU, percent) of the same kernels, same keys: near 100 the kernel
# is bound by its vector ALU work rather than by HBM.
MEASURED_VALU_BUSY = {
    ("b64", "k_rows_split<4>", "stream-v5"): 22.2,
    ("b256_topk_topp", "k_rows_stream", "stream-v5"): 45.6,
    ("ragged", "k_rows_stream", "stream-v5"): 67.0,
    ("large", "k_rows_stream", "stream-v5"): 101.5,
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline_threads(w, budget_s: float, threads: int, early=False):
    """The oracle on the first sessions of the workload, run by `threads` host
    threads at once (ctypes releases the GIL during the oracle's C call), one
    block of sessions per call.  The sample is sized from one session's time so
    that the parallel section takes about budget_s."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    from token_sampling_amd import workloads as W

    oracle.lib()

    def run(h):
        oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"],
                      h["seed"], h["round"], diagnostics=False, early=early)

    h0 = W.to_numpy(w, sessions=[0])
    t0 = time.perf_counter()
    run(h0)
    per = max(time.perf_counter() - t0, 1e-6)
    n = int(min(w.B, max(threads, budget_s * threads / per)))
    blocks = np.array_split(np.arange(n), threads)
    hs = [W.to_numpy(w, sessions=list(bl)) for bl in blocks if len(bl)]
    positions = int(sum((np.asarray(h["m"], dtype=np.int64) + 1).sum() for h in hs))
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=len(hs)) as ex:
        list(ex.map(run, hs))
    elapsed = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": positions / elapsed,
        "unit": "positions/s",
        "cores": len(hs),
        "kind": "oracle",
        "sample": f"sessions 0..{n - 1} of {w.name} (P={positions}) in {len(hs)} blocks, "
                  f"{elapsed:.1f} s on {len(hs)} host threads ({model})"
                  + (", read in order" if early else ""),
    }


def cpu_baseline(w, budget_s: float, sdcp_raw=None, q_rows=None, early=False):
    """Time the oracle on the first sessions of the workload (bounded sample).
    sdcp_raw: the [B, 32] session records (numpy uint8) when SDCP values are used;
    q_rows: the [B, M, V] published draft rows (device tensor) in q-rows mode;
    early: the oracle's in-order reading (rows after the deciding position unread)."""
    import numpy as np

    import oracle
    from token_sampling_amd import workloads as W

    sdcp = None if sdcp_raw is None else \
        np.ascontiguousarray(sdcp_raw).view(oracle.SDCP_SESSION_DTYPE).reshape(-1)

    oracle.lib()
    n = 1
    done_sessions = 0
    positions = 0
    elapsed = 0.0
    while done_sessions < w.B and elapsed < budget_s:
        idx = list(range(done_sessions, min(w.B, done_sessions + n)))
        h = W.to_numpy(w, sessions=idx)
        qh = None
        if q_rows is not None:
            qh = q_rows[idx[0]:idx[-1] + 1].cpu().numpy()
            h["draft"] = None
        t0 = time.perf_counter()
        oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"],
                      h["seed"], h["round"], diagnostics=False,
                      sdcp_sessions=None if sdcp is None else sdcp[idx], q_rows=qh, early=early)
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
                  f"{elapsed:.1f} s single-threaded" + (", read in order" if early else ""),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--logits", choices=("bf16", "fp32"), default=None,
                    help="store the workload's logits as bf16 or binary32 (default: the "
                         "workload's own type)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--cpu-threads", type=int, default=1,
                    help="host threads for the CPU baseline (1: the oracle as defined, one "
                         "core; N: blocks of sessions on N threads at once, Philox values "
                         "and draft logits only)")
    ap.add_argument("--sessions", type=int, default=None,
                    help="diagnostic only: the workload's first N sessions instead of all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain elementwise copy kernel "
                         "(1 GiB read, 1 GiB written) three times, to calibrate HBM "
                         "byte counters under a profiler")
    ap.add_argument("--sdcp", action="store_true",
                    help="time sv_verify_sdcp: the SDCP HMAC-SHA-256 verifier values from "
                         "per-session records (seeded random ids and seeds) instead of Philox")
    ap.add_argument("--qrows", action="store_true",
                    help="time sv_verify_qrows: draft distributions as published binary32 rows "
                         "(the synthetic drafter's own distribution) instead of draft logits")
    ap.add_argument("--early", type=int, default=None, metavar="W",
                    help="time sv_verify_early: positions read in order, in windows of W, 2W, "
                         "4W, ... positions, each only for the sessions still undecided")
    ap.add_argument("--commit", action="store_true",
                    help="add the commit step (sv_commit: truncation, digest chain, counters) "
                         "to every step, with per-session state carried across steps")
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
    w = W.make(args.workload, device="cuda", sessions=args.sessions, logits=args.logits)
    smp = w.sampling_tensor(dev)
    B, M, V = w.B, w.M, w.V
    P = w.positions()
    ws = torch.empty(sv.workspace_bytes(B, M, V), dtype=torch.uint8, device=dev)
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty((B, M + 1), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream(dev)
    sdcp = None
    if args.sdcp:
        import numpy as np

        ids = np.random.default_rng(w.seed & 0xFFFFFFFF).integers(0, 256, (B, 16), dtype=np.uint8)
        sdcp = sv.make_sdcp_sessions(B, seed=w.seed, round_=w.round, session_ids=ids, device=dev)

    q_rows = w.drafter_q_rows() if args.qrows else None
    draft = None if args.qrows else w.draft

    contracts = states = cres = None
    if args.commit:
        contracts = sv.make_contracts(B, m_max=M, max_new=1 << 30, low_rounds=3, stop=(),
                                      device=dev)
        states = sv.make_states(B, m_cap=M, device=dev)
        cres = {"emitted_len": torch.empty(B, dtype=torch.int32, device=dev),
                "action": torch.empty(B, dtype=torch.int32, device=dev)}

    def step(ev=None):
        sv.verify(w.target, draft, w.tokens, w.m, w.rule, smp, w.seed, w.round,
                  workspace=ws, out=out, stream=stream, row_events=ev, sdcp_sessions=sdcp,
                  q_rows=q_rows, early=args.early)
        if args.commit:
            sv.commit(contracts, states, w.m, out["accepted_len"], out["out_tokens"],
                      stream=stream, out=cres)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    # bf16 rows are all taken by the single-pass kernel: two events bracket it;
    # fp32 rows go to the generic kernel: a third event between the two.  Read
    # in order, two events bracket all the windows' row and advance kernels.
    bf16 = w.target.dtype == torch.bfloat16
    n_ev = 2 if (bf16 or args.early) else 3
    row_ev = [tuple(sv.HipEvent() for _ in range(n_ev)) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    # the timed region: exactly K steps, with no event inside a step (an event
    # recorded between two kernels of a step adds about 5 us to it)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    # then K more steps, outside the timed region, with HIP events around the
    # row kernels for the roofline line
    for k in range(args.steps):
        step(row_ev[k])
    torch.cuda.synchronize()
    stream_ms = sum(e[0].elapsed_ms(e[1]) for e in row_ev) / args.steps
    generic_ms = 0.0 if n_ev == 2 else sum(e[1].elapsed_ms(e[2]) for e in row_ev) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step, single-pass row kernel "
        f"{stream_ms:.4f} ms, generic row kernel {generic_ms:.4f} ms")

    # the dominant kernel: the row kernel that takes longer; its algorithmic
    # bytes are the rows it handles
    split = w.row_bytes_by_kernel(q_rows=args.qrows)
    kname, kms, kbytes = (("k_rows_stream", stream_ms, split["stream"]) if stream_ms >= generic_ms
                          else ("k_rows_generic", generic_ms, split["generic"]))
    if kname == "k_rows_stream" and B * (M + 1) + (B * M if draft is not None else 0) < 1024:
        kname = "k_rows_split<4>"  # launches under 1024 row slots split each row over 4 waves
    a = out["accepted_len"].cpu()
    if args.early:
        # read in order, the rows a session needs are its first a+1 target rows
        # and (rule 2 with draft logits) as many draft rows; failed sessions are
        # counted as reading nothing
        import numpy as np

        an = a.numpy().astype(np.int64)
        ok = an >= 0
        e = an + 1
        mm = w.m.cpu().numpy().astype(np.int64)
        r2 = w.rule.cpu().numpy() == sv.RULE_SPECULATIVE
        rows_needed = e[ok].sum()
        if not args.qrows:
            rows_needed += np.minimum(e, mm)[ok & r2].sum()
        kname = "row kernels, all windows"
        kms = stream_ms + generic_ms
        kbytes = int(rows_needed) * V * w.target.element_size()
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x (1 GiB read + 1 GiB written)")

    achieved = kbytes / (kms * 1e-3) / 1e9
    measured = not (args.sdcp or args.qrows or args.early or args.sessions)
    traffic = MEASURED_TRAFFIC.get((args.workload, kname, KERNEL_REVISION)) if measured else None
    valu_busy = MEASURED_VALU_BUSY.get((args.workload, kname, KERNEL_REVISION)) if measured else None
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
            "uniforms": "sdcp-hmac-sha256" if args.sdcp else "philox4x64-10",
            "draft": "q_rows fp32" if args.qrows else "logits",
            "commit_step": bool(args.commit),
            "reading": f"in order, first window {args.early}" if args.early else "every row",
            "positions_per_step": P, "algorithmic_bytes_per_step": w.algorithmic_bytes(q_rows=args.qrows),
            "mean_accepted": float(a[a >= 0].float().mean()) if (a >= 0).any() else None,
            "bad_proposals": int((a == sv.S_BAD_PROPOSAL).sum()),
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "valu_busy_pct": valu_busy,
            "kernel": kname, "ms_per_launch": kms, "algorithmic_bytes_per_launch": kbytes,
            "row_kernels_ms": {"k_rows_stream": stream_ms, "k_rows_generic": generic_ms},
        },
    }
    if args.cpu_budget > 0:
        log(f"[bench] oracle CPU baseline (~{args.cpu_budget:.0f} s)")
        if args.cpu_threads > 1 and sdcp is None and q_rows is None:
            result["cpu_baseline"] = cpu_baseline_threads(w, args.cpu_budget, args.cpu_threads,
                                                          early=bool(args.early))
        else:
            result["cpu_baseline"] = cpu_baseline(
                w, args.cpu_budget, None if sdcp is None else sdcp.cpu().numpy(), q_rows,
                early=bool(args.early))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
