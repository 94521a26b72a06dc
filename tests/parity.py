"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same host inputs and compare them element by element.

Bar (the acceptance step's stated tolerance): accepted_len and out_tokens
bit-identical, except in a session whose oracle diagnostics show a decision
within 1e-6 of its threshold (an acceptance test |u - min(1, p/q)|, a top-p
boundary |1000*C - P*Z_k| / (1000*Z_k), or an inverse-CDF boundary); such
sessions are counted and reported.  Probabilities p_i(x_i), q_i(x_i) agree
within 1e-5 relative.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import token_sampling_amd as sv

NEAR_TIE = 1e-6
PROB_RTOL = 1e-5


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


def random_sdcp_sessions(B, rng):
    """Random 16-octet ids, 64-bit seeds and rounds per session."""
    s = np.zeros(B, dtype=oracle.SDCP_SESSION_DTYPE)
    s["id"] = rng.integers(0, 256, size=(B, 16), dtype=np.uint8)
    s["seed"] = rng.integers(0, 1 << 63, size=B, dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=B, dtype=np.uint64)
    s["round"] = rng.integers(1, 1 << 32, size=B, dtype=np.uint64).astype(np.uint32)
    return s


def session_near_tie(o, b):
    vals = [o["d_acc"][b].min(), o["d_topp_t"][b].min(), o["d_topp_d"][b].min(), o["d_cdf"][b]]
    return float(min(vals))


def compare(g, o, label=""):
    """Return a report dict; raises AssertionError on an unexcused mismatch."""
    B = o["accepted_len"].shape[0]
    mism, excused = [], []
    for b in range(B):
        same = (g["accepted_len"][b] == o["accepted_len"][b]
                and np.array_equal(g["out_tokens"][b], o["out_tokens"][b]))
        if same:
            continue
        d = session_near_tie(o, b)
        (excused if d < NEAR_TIE else mism).append((b, d))
    max_rel = 0.0
    prob_bad = []
    if "p_tok" in g:
        for name in ("p_tok", "q_tok"):
            gp, op = g[name], o[name]
            for b in range(B):
                if any(e[0] == b for e in excused):
                    continue
                ok_rows = op[b] >= 0
                both = ok_rows & (op[b] > 0) & (gp[b] > 0)
                if both.any():
                    rel = np.abs(gp[b][both] - op[b][both]) / op[b][both]
                    max_rel = max(max_rel, float(rel.max()))
                    if (rel > PROB_RTOL).any():
                        prob_bad.append((name, b, float(rel.max())))
                zero_mismatch = ok_rows & ((op[b] > 0) != (gp[b] > 0))
                if zero_mismatch.any() and session_near_tie(o, b) >= NEAR_TIE:
                    prob_bad.append((name, b, "support"))
                neg_mismatch = (op[b] < 0) != (gp[b] < 0)
                if neg_mismatch.any():
                    prob_bad.append((name, b, "defined"))
    a = o["accepted_len"]
    rep = dict(label=label, sessions=B, ok_sessions=int((a >= 0).sum()),
               mean_a=float(a[a >= 0].mean()) if (a >= 0).any() else None,
               bad_proposal=int((a == oracle.S_BAD_PROPOSAL).sum()),
               excused_near_ties=len(excused), max_prob_rel=max_rel)
    log(f"[parity] {rep}")
    detail = [(b, d, int(g["accepted_len"][b]), int(o["accepted_len"][b]),
               g["out_tokens"][b].tolist(), o["out_tokens"][b].tolist()) for b, d in mism[:5]]
    assert not mism, (f"{label}: unexcused mismatches (session, near-tie distance, gpu a, "
                      f"oracle a, gpu tokens, oracle tokens): {detail}")
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
