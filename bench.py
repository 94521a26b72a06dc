#!/usr/bin/env python3
"""Benchmark of the verifier acceptance step (libspecverify) on one MI355X.

A step is one sv_verify call (sv_verify_sdcp with --sdcp, sv_verify_qrows with
--qrows, sv_verify_early with --early W) over one batch of synthetic logits
already resident in HBM: the single-pass row kernel (session checks and the row
profiles, the HBM-streaming part), the binary32 cut-row kernel (binary32 rows
with top-p or top-k above 64), and the per-session
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

# Counter readings of the row kernels (HBM bytes per launch from rocprofv3
# FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy; VALU busy percent), kept
# in profiles/counters.json under a hash of the row kernels' sources: a reading
# is reported only while the sources it was taken on are unchanged.
COUNTERS_FILE = os.path.join(HERE, "profiles", "counters.json")
ROW_KERNEL_SOURCES = ("sv_rows_stream.hip", "sv_rows_topk.hpp", "sv_rows_topk32.hpp",
                      "sv_rows_dense.hpp", "sv_rows_exact.hpp", "sv_stream.hpp", "sv_common.hpp",
                      "sv_kernels.hpp", "sv_sdcp.hpp", "sv_commit.hpp")
CONFIG_NAMES = ("tiny", "b64", "b256_topk_topp", "ragged", "large")


def row_kernel_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in ROW_KERNEL_SOURCES:
        with open(os.path.join(HERE, "token_sampling_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def kernel_short_name(full: str) -> str:
    import re

    m = re.search(r"(k_rows_stream|k_rows_split<\d+>|k_rows_dense32|k_finalize|k_advance|k_commit)",
                  full)
    return m.group(1) if m else ""


def ingest_counters(root: str) -> dict:
    """Counter passes of this benchmark, as rocprofv3 --pmc writes them: under
    root, for each workload W, fetch_W, write_W and valu_W (FETCH_SIZE,
    WRITE_SIZE and VALUBusy, one pass each, every run with --copy-calibration
    for the first two).  Bytes per dispatch are scaled by what the same counter
    reads for the calibration copy (torch.neg over 2^28 float32: 1 GiB read,
    1 GiB written); each kernel's figure is the median over its dispatches
    after the first.  Returns {W: {kernel: {...}}}."""
    import csv
    import glob
    import statistics

    def passes(kind, w):
        files = glob.glob(os.path.join(root, f"{kind}_{w}", "**", "*counter_collection.csv"),
                          recursive=True)
        per = {}
        for fn in files:
            with open(fn) as f:
                for r in csv.DictReader(f):
                    per.setdefault((r["Kernel_Name"], int(r["Dispatch_Id"])), 0.0)
                    per[(r["Kernel_Name"], int(r["Dispatch_Id"]))] += float(r["Counter_Value"])
        by_kernel = {}
        for (name, disp), v in sorted(per.items(), key=lambda kv: kv[0][1]):
            by_kernel.setdefault(name, []).append(v)
        return by_kernel

    out = {}
    for w in CONFIG_NAMES:
        fetch, write, valu = passes("fetch", w), passes("write", w), passes("valu", w)
        if not fetch or not write:
            continue

        def copy_value(table):
            # the calibration's three dispatches are the largest of torch.neg's
            # (the workload's construction also negates small tensors)
            vals = sorted(v for name, vs in table.items() if "neg_kernel" in name for v in vs)
            return statistics.median(vals[-3:]) if len(vals) >= 3 else None

        fcopy, wcopy = copy_value(fetch), copy_value(write)
        if not fcopy or not wcopy:
            continue
        fscale, wscale = (1 << 20) / fcopy, (1 << 20) / wcopy
        rec = {}
        for name, vs in fetch.items():
            short = kernel_short_name(name)
            if not short:
                continue
            fk = statistics.median(vs[1:] or vs)
            wk = statistics.median((write.get(name) or [0.0])[1:] or write.get(name) or [0.0])
            ent = {"fetch_kib": fk, "write_kib": wk, "fetch_scale": fscale, "write_scale": wscale,
                   "traffic": int(round(fk * 1024 * fscale + wk * 1024 * wscale))}
            vv = valu.get(name)
            if vv:
                ent["valu_busy_pct"] = statistics.median(vv[1:] or vv)
            rec[short] = ent
        out[w] = rec
    return out


def counter_record(workload: str):
    """The counters recorded for this workload under the current row-kernel
    sources, or None."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec.get(row_kernel_hash(), {}).get(workload)


def counters_for(workload: str, kname: str):
    rec = counter_record(workload)
    return (rec or {}).get(kname)


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


def measure(w, args, sv, torch, draft, q_rows=None, sdcp=None, early=None, commit=False,
            scrub=False):
    """Time one workload on the GPU: W warm-up steps, then K timed steps (one
    sv_verify* call each), then K more steps with HIP events around the row
    kernels.  scrub: inputs small enough to stay in the 256 MB last-level
    cache are timed step by step with a 1 GiB write between steps (outside the
    step's events), so that every step reads its rows from HBM.  Returns the
    step time, the row kernels' times and the last step's outputs (host)."""
    dev = w.target.device
    B, M, V = w.B, w.M, w.V
    smp = w.sampling_tensor(dev)
    ws = torch.empty(sv.workspace_bytes(B, M, V), dtype=torch.uint8, device=dev)
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty((B, M + 1), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream(dev)
    contracts = states = cres = None
    if commit:
        contracts = sv.make_contracts(B, m_max=M, max_new=1 << 30, low_rounds=3, stop=(),
                                      device=dev)
        states = sv.make_states(B, m_cap=M, device=dev)
        cres = {"emitted_len": torch.empty(B, dtype=torch.int32, device=dev),
                "action": torch.empty(B, dtype=torch.int32, device=dev)}

    # the commit step: inside the call (sv_verify_commit) where it can be, else
    # sv_commit after the acceptance step
    joint = commit and q_rows is None and early is None
    if joint:
        out.update(cres)

    def step(ev=None):
        sv.verify(w.target, draft, w.tokens, w.m, w.rule, smp, w.seed, w.round,
                  workspace=ws, out=out, stream=stream, row_events=ev, sdcp_sessions=sdcp,
                  q_rows=q_rows, early=early,
                  commit=(contracts, states, None) if joint else None)
        if commit and not joint:
            sv.commit(contracts, states, w.m, out["accepted_len"], out["out_tokens"],
                      stream=stream, out=cres)

    junk = torch.empty(1 << 28, dtype=torch.float32, device=dev) if scrub else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # bf16 rows are all taken by the single-pass kernel: two events bracket it;
    # binary32 rows may also take the cut-row kernel: a third event between
    # the two.  Read in order, two events bracket all the windows' row and advance
    # kernels.
    n_ev = 2 if (w.target.dtype == torch.bfloat16 or early) else 3
    row_ev = [tuple(sv.HipEvent() for _ in range(n_ev)) for _ in range(args.steps)]
    if scrub:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for k in range(args.steps):
            junk.fill_(float(k))
            ev[k][0].record(stream)
            step()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        ms_per_step = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    else:
        # the timed region: exactly K steps, with no event inside a step (an
        # event recorded between two kernels of a step adds about 5 us to it)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(stop) / args.steps
    for k in range(args.steps):
        if scrub:
            junk.fill_(float(k))
        step(row_ev[k])
    torch.cuda.synchronize()
    stream_ms = sum(e[0].elapsed_ms(e[1]) for e in row_ev) / args.steps
    dense32_ms = 0.0 if n_ev == 2 else sum(e[1].elapsed_ms(e[2]) for e in row_ev) / args.steps
    del junk
    return {"ms_per_step": ms_per_step, "stream_ms": stream_ms, "dense32_ms": dense32_ms,
            "accepted_len": out["accepted_len"].cpu().numpy(),
            "out_tokens": out["out_tokens"].cpu().numpy()}


def roofline(w, r, qrows=False, early=False):
    """The dominant row kernel's algorithmic rate: the bytes of the rows it
    handles, each once, over its average duration (HIP events on the launch
    stream)."""
    import numpy as np

    B, M = w.B, w.M
    split = w.row_bytes_by_kernel(q_rows=qrows)
    stream_ms, dense32_ms = r["stream_ms"], r["dense32_ms"]
    kname, kms, kbytes = (("k_rows_stream", stream_ms, split["stream"]) if stream_ms >= dense32_ms
                          else ("k_rows_dense32", dense32_ms, split["dense32"]))
    rows = B * (M + 1) + (B * M if not qrows else 0)
    if kname == "k_rows_stream" and w.target.dtype.itemsize == 2 and rows < 1024:
        kname = "k_rows_split<4>"  # bf16 launches under 1024 row slots split each row
    if early:
        # read in order, the rows a session needs are its first a+1 target rows
        # and (rule 2 with draft logits) as many draft rows; failed sessions are
        # counted as reading nothing
        an = r["accepted_len"].astype(np.int64)
        ok = an >= 0
        e = an + 1
        mm = w.m.cpu().numpy().astype(np.int64)
        r2 = w.rule.cpu().numpy() == 2
        rows_needed = e[ok].sum()
        if not qrows:
            rows_needed += np.minimum(e, mm)[ok & r2].sum()
        kname = "row kernels, all windows"
        kms = stream_ms + dense32_ms
        kbytes = int(rows_needed) * w.V * w.target.element_size()
    achieved = kbytes / (kms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "kernel": kname, "ms_per_launch": kms,
            "algorithmic_bytes_per_launch": kbytes,
            "row_kernels_ms": {"k_rows_stream": stream_ms, "k_rows_dense32": dense32_ms}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def oracle_config(w, gpu, budget_1core: float):
    """The oracle (run unchanged) on this workload: single-threaded on its first
    sessions for about budget_1core seconds, then over every session on the
    host's threads (at most 16; B=1024, M=64: the oracle's in-order reading,
    which gives the same verdicts where every row is usable), with the GPU's
    accepted_len and out_tokens compared session by session."""
    import contextlib

    from tests import parity

    one = cpu_baseline(w, budget_1core) if budget_1core > 0 else None
    early = w.name == "large"
    threads = parity.host_threads()
    t0 = time.perf_counter()
    o = parity.run_oracle_sessions(w, early=early)
    elapsed = time.perf_counter() - t0
    with contextlib.redirect_stdout(sys.stderr):  # stdout carries the one JSON line
        rep = parity.compare({"accepted_len": gpu["accepted_len"],
                              "out_tokens": gpu["out_tokens"]}, o, w.name, strict=False)
    P = w.positions()
    return {
        "oracle_1core_positions_per_s": None if one is None else one["value"],
        "oracle_all_positions_per_s": P / elapsed,
        "oracle_threads": threads,
        "oracle_reading": "in order" if early else "every row",
        "sessions_checked": rep["sessions"], "mismatches": rep["mismatches"],
        "excused_by_kind": rep["excused"], "near_ties_by_kind": rep["near_ties"],
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
    ap.add_argument("--configs", choices=("all", "none"), default=None,
                    help="also time the five workloads and check them against the oracle "
                         "(default: all, unless a single-workload option is given)")
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
                    help="time sv_verify_early: positions read in order, in windows of W, 4W, "
                         "16W, ... positions, each only for the sessions still undecided")
    ap.add_argument("--commit", action="store_true",
                    help="add the commit step (truncation, digest chain, counters) to every "
                         "step, with per-session state carried across steps: sv_verify_commit "
                         "(sv_commit after the call with --qrows or --early)")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="read rocprofv3 counter passes under DIR (fetch_W, write_W, valu_W) and "
                         "record them in profiles/counters.json under the current row-kernel "
                         "sources; no GPU work")
    args = ap.parse_args()

    if args.ingest_counters:
        rec = ingest_counters(args.ingest_counters)
        try:
            with open(COUNTERS_FILE) as f:
                allrec = json.load(f)
        except (OSError, ValueError):
            allrec = {}
        allrec.setdefault(row_kernel_hash(), {}).update(rec)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(allrec, f, indent=1, sort_keys=True)
        print(json.dumps({"sources": row_kernel_hash(), "workloads": sorted(rec)}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the verifier step shards by session with no exchange, so N GPUs run N "
              "independent copies of this single-GPU step.", file=sys.stderr)
        sys.exit(2)
    single = (args.sdcp or args.qrows or args.early or args.commit or args.sessions or
              args.logits or args.copy_calibration or args.workload != DEFAULT_WORKLOAD)
    run_configs = (args.configs == "all") or (args.configs is None and not single)

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
    B, M, V = w.B, w.M, w.V
    P = w.positions()
    sdcp = None
    if args.sdcp:
        import numpy as np

        ids = np.random.default_rng(w.seed & 0xFFFFFFFF).integers(0, 256, (B, 16), dtype=np.uint8)
        sdcp = sv.make_sdcp_sessions(B, seed=w.seed, round_=w.round, session_ids=ids, device=dev)
    q_rows = w.drafter_q_rows() if args.qrows else None
    draft = None if args.qrows else w.draft

    r = measure(w, args, sv, torch, draft, q_rows=q_rows, sdcp=sdcp, early=args.early,
                commit=args.commit)
    log(f"[bench] {args.steps} steps: {r['ms_per_step']:.4f} ms/step, single-pass row kernel "
        f"{r['stream_ms']:.4f} ms, binary32 cut-row kernel {r['dense32_ms']:.4f} ms")
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x (1 GiB read + 1 GiB written)")

    roof = roofline(w, r, qrows=args.qrows, early=args.early)
    rec = None if (args.sdcp or args.qrows or args.early or args.sessions or args.logits) \
        else counters_for(args.workload, roof["kernel"])
    roof["traffic"] = rec.get("traffic") if rec else None
    roof["valu_busy_pct"] = rec.get("valu_busy_pct") if rec else None
    roof["counters_for_sources"] = row_kernel_hash()
    a = r["accepted_len"]
    result = {
        "metric": METRIC,
        "value": P / (r["ms_per_step"] * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
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
            "commit_step": (False if not args.commit else
                            "sv_commit after the call" if (args.qrows or args.early)
                            else "in the call (sv_verify_commit)"),
            "reading": f"in order, first window {args.early}" if args.early else "every row",
            "positions_per_step": P,
            "algorithmic_bytes_per_step": w.algorithmic_bytes(q_rows=args.qrows),
            "mean_accepted": float(a[a >= 0].mean()) if (a >= 0).any() else None,
            "bad_proposals": int((a == sv.S_BAD_PROPOSAL).sum()),
        },
        "roofline": roof,
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
            if run_configs:
                from tests import parity

                result["cpu_baseline"]["all_cores"] = cpu_baseline_threads(
                    w, max(2.0, args.cpu_budget / 3), parity.host_threads())
    else:
        result["cpu_baseline"] = None

    if run_configs:
        configs = {}
        del w, draft, q_rows, r
        torch.cuda.empty_cache()
        for name in CONFIG_NAMES:
            log(f"[bench] config {name}")
            wc = W.make(name, device="cuda")
            small = wc.algorithmic_bytes() < (1 << 30)
            rc = measure(wc, args, sv, torch, wc.draft, scrub=small)
            roofc = roofline(wc, rc)
            recc = counters_for(name, roofc["kernel"])
            ac = rc["accepted_len"]
            Pc = wc.positions()
            ent = {
                "B": wc.B, "M": wc.M, "V": wc.V,
                "logits": "bf16" if wc.target.dtype == torch.bfloat16 else "fp32",
                "positions_per_step": Pc, "ms_per_step": rc["ms_per_step"],
                "positions_per_s": Pc / (rc["ms_per_step"] * 1e-3),
                "algorithmic_bytes_per_step": wc.algorithmic_bytes(),
                "step_gbs": wc.algorithmic_bytes() / (rc["ms_per_step"] * 1e-3) / 1e9,
                "step_frac": wc.algorithmic_bytes() / (rc["ms_per_step"] * 1e-3) / 1e9
                / HBM_PEAK_GBS,
                "cold_hbm": "1 GiB written between steps" if small else "inputs exceed the cache",
                "row_kernel": roofc["kernel"], "row_kernel_ms": roofc["ms_per_launch"],
                "row_kernel_gbs": roofc["achieved"], "row_kernel_frac": roofc["frac"],
                "traffic": recc.get("traffic") if recc else None,
                "valu_busy_pct": recc.get("valu_busy_pct") if recc else None,
                "mean_accepted": float(ac[ac >= 0].mean()) if (ac >= 0).any() else None,
                "bad_proposals": int((ac == sv.S_BAD_PROPOSAL).sum()),
            }
            if args.cpu_budget > 0:
                ent.update(oracle_config(wc, rc, budget_1core=min(5.0, args.cpu_budget / 3)))
            configs[name] = ent
            log(f"[bench] {name}: {json.dumps(ent)}")
            del wc, rc
            torch.cuda.empty_cache()
        result["configs"] = configs
        result["host"] = {"cpu_model": cpu_model(), "cpu_count": os.cpu_count()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
