"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same host inputs and compare them element by element.

Bar (the acceptance step's stated tolerance): accepted_len and out_tokens
bit-identical.  A session that differs is excused only when the first decision
at which it departs from the oracle lies within 1e-6 of its threshold, as the
oracle measured it:
  - an acceptance test at position i: |u - min(1, p/q)|;
  - a top-p cut of a row that decision reads: |1000*C - P*Z_k| / (1000*Z_k);
  - the inverse CDF of the additional token: distance of u*S to the nearest
    CDF boundary around the pick, over S.
Excused sessions and near-ties are counted by kind and reported.
Probabilities p_i(x_i), q_i(x_i) agree within 1e-5 relative (1e-5 is the
stated bound; callers may ask for a tighter one), except in a row whose top-p
cut the oracle found within 1e-6 of its threshold: there the support, and so
the normaliser, may differ by the tokens at the cut (counted and reported).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle
import token_sampling_amd as sv

NEAR_TIE = 1e-6
PROB_RTOL = 1e-5
# the dense path's probabilities at the true temperature (binary64 weights, Z
# from a binary32 pass with its scale and window corrected): well inside the
# acceptance test's 1e-6 near-tie band
DENSE_PROB_RTOL = 2e-7
KINDS = ("acc", "topp", "cdf")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def sampling_bytes(s, device="cuda"):
    raw = np.ascontiguousarray(s, dtype=oracle.SAMPLING_DTYPE).view(np.uint8).reshape(len(s), 24)
    return torch.from_numpy(raw.copy()).to(device)


def sdcp_bytes(sess, device="cuda"):
    """[B] records of oracle.SDCP_SESSION_DTYPE as the library's 32-byte records."""
    raw = np.ascontiguousarray(sess, dtype=oracle.SDCP_SESSION_DTYPE).view(np.uint8).reshape(len(sess), 32)
    return torch.from_numpy(raw.copy()).to(device)


def run_gpu(h, probe=True, device="cuda"):
    """h["sdcp"] (optional): [B] oracle.SDCP_SESSION_DTYPE records -> sv_verify_sdcp;
    h["q_rows"] (optional): [B, M, V] float32 published draft rows -> sv_verify_qrows."""
    t = to_device(h["target"], device)
    d = to_device(h["draft"], device)
    q = h.get("q_rows")
    sess = h.get("sdcp")
    out = sv.verify(t, d, to_device(np.asarray(h["tokens"], np.int32), device),
                    to_device(np.asarray(h["m"], np.int32), device),
                    to_device(np.asarray(h["rule"], np.int32), device),
                    sampling_bytes(h["sampling"], device), h["seed"], h["round"], probe=probe,
                    sdcp_sessions=None if sess is None else sdcp_bytes(sess, device),
                    q_rows=None if q is None else to_device(np.asarray(q, np.float32), device),
                    early=h.get("early"))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def run_oracle(h, diagnostics=True):
    return oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"],
                         h["seed"], h["round"], diagnostics=diagnostics,
                         sdcp_sessions=h.get("sdcp"), q_rows=h.get("q_rows"),
                         early=h.get("early") is not None)


def host_threads():
    """Threads for the oracle: the host's cores, at most 16 (one GPU's share of
    a shared host)."""
    env = os.environ.get("SV_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def run_oracle_sessions(w, sessions=None, early=False, diagnostics=True, threads=None,
                        block=None, extra=None):
    """The oracle, unchanged, over the given sessions of a workload held on the
    GPU (all by default), in blocks of sessions on host threads (the C call
    releases the GIL).  Blocks are copied to the host one at a time, at most
    two more than the threads ahead of the oracle, so host memory stays
    bounded.  Returns
    the oracle's arrays stacked in session order.  extra(ids, h), if given,
    edits a block's host inputs h (sessions ids) before the oracle runs (q
    rows, SDCP records, another rule)."""
    from token_sampling_amd import workloads as W

    idx = np.arange(w.B) if sessions is None else np.asarray(sessions, dtype=np.int64)
    threads = threads or host_threads()
    if block is None:
        block = max(1, min(32, -(-len(idx) // (2 * threads))))
    blocks = [idx[i:i + block] for i in range(0, len(idx), block)]
    oracle.lib()
    oracle.sha256(b"")  # the oracle's SHA-256 constants, set up before the threads start

    def run(h):
        if early:
            h["early"] = 1
        return run_oracle(h, diagnostics=diagnostics)

    results = [None] * len(blocks)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        pending = {}
        for k, bl in enumerate(blocks):
            while len(pending) >= threads + 2:
                done, _ = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
                for f in done:
                    results[pending.pop(f)] = f.result()
            h = W.to_numpy(w, sessions=torch.as_tensor(bl, device=w.target.device))
            if extra is not None:
                extra(bl, h)
            pending[ex.submit(run, h)] = k
        for f in cf.as_completed(list(pending)):
            results[pending[f]] = f.result()
    return {key: np.concatenate([r[key] for r in results], axis=0) for key in results[0]}


def random_sdcp_sessions(B, rng):
    """Random 16-octet ids, 64-bit seeds and rounds per session."""
    s = np.zeros(B, dtype=oracle.SDCP_SESSION_DTYPE)
    s["id"] = rng.integers(0, 256, size=(B, 16), dtype=np.uint8)
    s["seed"] = rng.integers(0, 1 << 63, size=B, dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=B, dtype=np.uint64)
    s["round"] = rng.integers(1, 1 << 32, size=B, dtype=np.uint64).astype(np.uint32)
    return s


def _row_delta(o, name, b, i):
    arr = o.get(name)
    if arr is None or i < 0 or i >= arr.shape[1]:
        return np.inf
    return float(arr[b, i])


def first_difference(g, o, b):
    """(delta, kind) of the first decision at which the GPU's session b departs
    from the oracle's; (inf, None) when no decision within reach of rounding
    can explain the difference (a status other than a bad proposal, or a
    decision far from its threshold).

    The oracle decides positions in order: position i's top-p cuts (target row
    i, draft row i) give p_i(x_i), q_i(x_i), then its acceptance test; at the
    first rejection (or after m acceptances) the additional token's inverse
    CDF over the row(s) it reads.  Positions before min(a_gpu, a_oracle) were
    accepted on both sides, so the first differing decision lies at that
    position.  Where the probes show x_i inside the support on one side and
    outside it on the other, the decision is that row's top-p cut; otherwise
    it is the acceptance test.  A differing additional token with equal a is
    the inverse CDF, or a top-p cut of a row the draw reads."""
    ag, ao = int(g["accepted_len"][b]), int(o["accepted_len"][b])
    has_probe = "p_tok" in g and "p_tok" in o
    if ag < 0 or ao < 0:
        # only a bad proposal can follow from rounding: q_i(x_i) = 0 on one side
        # because x_i sits at the top-p cut of its draft row
        if (ag < 0 and ag != oracle.S_BAD_PROPOSAL) or (ao < 0 and ao != oracle.S_BAD_PROPOSAL):
            return np.inf, None
        # a failed session's probes hold -1 on both sides, so the position is
        # not known: the closest draft-row cut of the session stands for it
        # (the oracle keeps the deltas of the rows it profiled)
        d = float(o["d_topp_d"][b].min()) if "d_topp_d" in o else np.inf
        return d, "topp"
    i = min(ag, ao)
    if ag != ao:
        kind, d = "acc", _row_delta(o, "d_acc", b, i)
        if has_probe and i < g["p_tok"].shape[1]:
            gp, op = g["p_tok"][b, i], o["p_tok"][b, i]
            gq, oq = g["q_tok"][b, i], o["q_tok"][b, i]
            dt = []
            if (gp > 0) != (op > 0):
                dt.append(_row_delta(o, "d_topp_t", b, i))
            if (gq > 0) != (oq > 0):
                dt.append(_row_delta(o, "d_topp_d", b, i))
            if dt:
                kind, d = "topp", min(dt)
        return d, kind
    # same a: the additional token's draw (inverse CDF), or a cut of its rows
    cands = [(float(o["d_cdf"][b]) if "d_cdf" in o else np.inf, "cdf"),
             (_row_delta(o, "d_topp_t", b, i), "topp"),
             (_row_delta(o, "d_topp_d", b, i), "topp")]
    return min(cands, key=lambda c: c[0])


def near_ties(o):
    """Decisions the oracle took within NEAR_TIE of their thresholds, by kind:
    acceptance tests at positions 1..min(a+1, m), top-p cuts of the rows those
    positions and the additional token read, the additional token's CDF."""
    out = {k: 0 for k in KINDS}
    if "d_acc" not in o:
        return out
    a = o["accepted_len"]
    B, M = o["d_acc"].shape
    for b in range(B):
        if a[b] < 0:
            continue
        n = int(a[b]) + 1  # positions examined (the last one decides)
        out["acc"] += int((o["d_acc"][b, :min(n, M)] < NEAR_TIE).sum())
        out["topp"] += int((o["d_topp_t"][b, :n] < NEAR_TIE).sum())
        out["topp"] += int((o["d_topp_d"][b, :min(n, M)] < NEAR_TIE).sum())
        out["cdf"] += int(o["d_cdf"][b] < NEAR_TIE)
    return out


def compare(g, o, label="", prob_rtol=PROB_RTOL, strict=True):
    """Return a report dict; raises AssertionError on an unexcused mismatch
    (strict; otherwise the report counts them)."""
    B = o["accepted_len"].shape[0]
    mism, excused = [], []
    for b in range(B):
        same = (g["accepted_len"][b] == o["accepted_len"][b]
                and np.array_equal(g["out_tokens"][b], o["out_tokens"][b]))
        if same:
            continue
        d, kind = first_difference(g, o, b)
        (excused if d < NEAR_TIE else mism).append((b, d, kind))
    excused_ids = {e[0] for e in excused}
    max_rel = 0.0
    prob_bad = []
    prob_at_cut = 0
    if "p_tok" in g:
        for name in ("p_tok", "q_tok"):
            gp, op = g[name], o[name]
            dname = "d_topp_t" if name == "p_tok" else "d_topp_d"
            for b in range(B):
                if b in excused_ids:
                    continue
                ok_rows = op[b] >= 0
                both = ok_rows & (op[b] > 0) & (gp[b] > 0)
                for i in np.nonzero(both)[0]:
                    rel = abs(gp[b, i] - op[b, i]) / op[b, i]
                    if rel <= prob_rtol:
                        max_rel = max(max_rel, float(rel))
                    elif _row_delta(o, dname, b, int(i)) < NEAR_TIE:
                        # the row's top-p cut is a near-tie: its support (so
                        # its normaliser) may hold a token more or less
                        prob_at_cut += 1
                    else:
                        max_rel = max(max_rel, float(rel))
                        prob_bad.append((name, b, int(i), float(rel)))
                # support membership: a difference is allowed only at a top-p cut
                # within NEAR_TIE (that row's oracle delta)
                for i in np.nonzero(ok_rows & ((op[b] > 0) != (gp[b] > 0)))[0]:
                    if _row_delta(o, dname, b, int(i)) >= NEAR_TIE:
                        prob_bad.append((name, b, int(i), "support"))
                neg_mismatch = (op[b] < 0) != (gp[b] < 0)
                if neg_mismatch.any():
                    prob_bad.append((name, b, "defined"))
    a = o["accepted_len"]
    by_kind = {k: sum(1 for e in excused if e[2] == k) for k in KINDS}
    rep = dict(label=label, sessions=B, ok_sessions=int((a >= 0).sum()),
               mean_a=float(a[a >= 0].mean()) if (a >= 0).any() else None,
               bad_proposal=int((a == oracle.S_BAD_PROPOSAL).sum()),
               mismatches=len(mism), excused=by_kind, near_ties=near_ties(o),
               max_prob_rel=max_rel, prob_at_near_tie_cut=prob_at_cut)
    log(f"[parity] {rep}")
    if not strict:
        return rep
    detail = [(b, d, k, int(g["accepted_len"][b]), int(o["accepted_len"][b]),
               g["out_tokens"][b].tolist(), o["out_tokens"][b].tolist()) for b, d, k in mism[:5]]
    assert not mism, (f"{label}: unexcused mismatches (session, delta of the first differing "
                      f"decision, kind, gpu a, oracle a, gpu tokens, oracle tokens): {detail}")
    assert not prob_bad, f"{label}: probability mismatches: {prob_bad[:10]}"
    return rep


def draw_valid_tokens(h, rng):
    """Draft tokens for rule-2 sessions drawn from q (the oracle's profile of the
    draft rows); greedy sessions get the draft argmax or a random token."""
    B, M = np.asarray(h["tokens"]).shape
    toks = np.zeros((B, M), dtype=np.int32)
    for b in range(B):
        s = h["sampling"][b]
        prof = (int(s["temperature_milli"]), int(s["top_k"]), int(s["top_p_milli"]))
        for i in range(M):
            row = h["draft"][b, i] if h["draft"] is not None else h["target"][b, i]
            if h["rule"][b] == 2 and h["draft"] is not None:
                st, q, _ = oracle.profile(row, *prof)
                if st != 0:
                    toks[b, i] = 0
                    continue
                toks[b, i] = rng.choice(q.shape[0], p=q / q.sum())
            else:
                toks[b, i] = int(rng.integers(0, row.shape[0])) if rng.random() < 0.3 else \
                    int(np.argmax(h["target"][b, i].astype(np.float32) if h["target"].dtype != np.uint16
                                  else oracle.bf16_to_float(h["target"][b, i])))
    return toks
