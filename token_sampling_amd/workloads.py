"""Seeded synthetic workloads for the verifier's acceptance step.

This module only draws inputs.  It holds none of the acceptance step's
arithmetic (no temperature/top-k/top-p profile, no acceptance test, no
residual): the GPU library and the oracle both receive what it produces, and
neither shares code with it beyond that.

Shapes follow the five workloads of the verifier acceptance step, named by
what they are (batch B, drafts per session M, vocabulary V).  The vocabulary
sizes match model families the pages mention: Llama-2 (32000), Llama-3
(128256), DeepSeek-V3 (129280); 151936 is the Qwen vocabulary.

Draft tokens.  For untruncated profiles (T > 0, no top-k, no top-p) each draft
token is drawn from softmax(draft_logits / T) with the Gumbel-max trick, which
is exactly q.  For truncated profiles a synthetic drafter proposes, by
Gumbel-max at temperature T, among the ids of its ``draft_top_n`` largest draft
logits (``torch.topk``); such a proposal can fall outside the verifier's
nucleus, and the verifier then reports it as a bad proposal.  Greedy (rule 1)
sessions of the ragged workload propose the draft argmax.

Published draft rows.  ``Workload.drafter_q_rows`` returns, as SDCP q_rows, the
distribution the synthetic drafter actually drew each token from: softmax at
temperature T over its top-n draft logits (or over all of them when the
profile is untruncated).  It is the drafter's arithmetic, not the verifier's
profile (no top-k / top-p cut of the session's profile is applied).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BF16 = 0
FP32 = 1

SAMPLING_DTYPE = np.dtype(
    [
        ("temperature_milli", "<u4"),
        ("top_k", "<u4"),
        ("top_p_milli", "<u4"),
        ("reserved", "<u4"),
        ("session_key", "<u8"),
    ],
    align=True,
)


@dataclasses.dataclass
class Workload:
    name: str
    target: torch.Tensor  # [B, M+1, V] bf16 or fp32
    draft: torch.Tensor | None  # [B, M, V]
    tokens: torch.Tensor  # [B, M] int32
    m: torch.Tensor  # [B] int32
    rule: torch.Tensor  # [B] int32
    sampling: np.ndarray  # [B] SAMPLING_DTYPE
    seed: int
    round: int

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def M(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def dtype_code(self):
        return BF16 if self.target.dtype == torch.bfloat16 else FP32

    def sampling_tensor(self, device) -> torch.Tensor:
        """The [B] sampling records as raw bytes on ``device`` (24 B each)."""
        raw = np.ascontiguousarray(self.sampling).view(np.uint8).reshape(self.B, 24)
        return torch.from_numpy(raw.copy()).to(device)

    def drafter_q_rows(self, draft_top_n: int = 8, chunk_sessions: int = 16) -> torch.Tensor:
        """[B, M, V] float32 rows: the synthetic drafter's distribution for each
        drafted position (what it publishes as q_rows).  Rows of greedy
        sessions are filled the same way; rule 1 never reads them."""
        B, M, V = self.B, self.M, self.V
        T = float(self.sampling["temperature_milli"][0]) / 1000.0
        untruncated = (int(self.sampling["top_k"][0]) == 0 and
                       int(self.sampling["top_p_milli"][0]) >= 1000)
        q = torch.zeros((B, M, V), dtype=torch.float32, device=self.draft.device)
        for s0 in range(0, B, chunk_sessions):
            d = self.draft[s0:s0 + chunk_sessions].float()
            if untruncated or draft_top_n >= V:
                q[s0:s0 + chunk_sessions] = torch.softmax(d / T, dim=-1)
            else:
                vals, ids = torch.topk(d, draft_top_n, dim=-1)
                q[s0:s0 + chunk_sessions].scatter_(-1, ids, torch.softmax(vals / T, dim=-1))
            del d
        return q

    def positions(self) -> int:
        """P = sum_b (m_b + 1): verified positions in one step."""
        m = self.m.to("cpu").to(torch.int64)
        return int((m + 1).sum())

    def algorithmic_bytes(self, q_rows: bool = False) -> int:
        """Bytes the step must move: each row a session's rule reads, once,
        plus the small per-session arrays and the outputs.  With q_rows the
        draft side is q_i(x_i) (4 B per drafted position) and, at most once
        per session, the residual's row (not counted: it depends on the draws)."""
        m = self.m.to("cpu").to(torch.int64)
        rule = self.rule.to("cpu").to(torch.int64)
        draft_rows = 0 if q_rows else int((m * (rule == 2)).sum())
        rows = int((m + 1).sum()) + draft_rows
        s = self.target.element_size()
        small = self.B * (4 * self.M + 4 + 4 + 24 + 4 + 4 * (self.M + 1))
        if q_rows:
            small += 4 * int((m * (rule == 2)).sum())
        return rows * self.V * s + small

    def row_bytes_by_kernel(self, q_rows: bool = False) -> dict:
        """Row bytes read by each row kernel: the single-pass kernel takes every
        bf16 row, and the binary32 rows of the top-k class (greedy rule,
        temperature 0, 1 <= top_k <= 64) or with temperature alone; the
        binary32 cut-row kernel the other binary32 rows (each counted once,
        though it reads the cut's coarse key in a second pass).  Rows a path
        hands back are not counted (that depends on the logits).  With q_rows
        no draft row is profiled."""
        m = self.m.to("cpu").to(torch.int64).numpy()
        rule = self.rule.to("cpu").to(torch.int64).numpy()
        per_session = (m + 1) + (0 if q_rows else m * (rule == 2))
        row = self.V * self.target.element_size()
        total = int(per_session.sum()) * row
        if self.target.dtype == torch.bfloat16:
            return {"stream": total, "dense32": 0}
        s = self.sampling
        topk_class = (rule == 1) | (s["temperature_milli"] == 0) | \
            ((s["top_k"] >= 1) & (s["top_k"] <= 64))
        untruncated = (s["top_p_milli"] >= 1000) & ((s["top_k"] == 0) | (s["top_k"] >= self.V))
        stream = int(per_session[topk_class | untruncated].sum()) * row
        return {"stream": stream, "dense32": total - stream}


def _to_storage(x32: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return x32.to(dtype)  # round to nearest even for bf16


def _gumbel_pick(logits: torch.Tensor, temperature: float, gen: torch.Generator,
                 top_n: int | None) -> torch.Tensor:
    """Gumbel-max draw over the last axis (optionally among the top_n ids)."""
    lf = logits.float()
    if top_n is not None and top_n < lf.shape[-1]:
        vals, ids = torch.topk(lf, top_n, dim=-1)
        u = torch.rand(vals.shape, generator=gen, device=lf.device).clamp_(1e-12, 1 - 1e-7)
        g = -torch.log(-torch.log(u))
        pick = torch.argmax(vals / temperature + g, dim=-1, keepdim=True)
        return torch.gather(ids, -1, pick).squeeze(-1).to(torch.int32)
    u = torch.rand(lf.shape, generator=gen, device=lf.device).clamp_(1e-12, 1 - 1e-7)
    g = -torch.log(-torch.log(u))
    return torch.argmax(lf / temperature + g, dim=-1).to(torch.int32)


def _sampling(B, t_milli, top_k, top_p_milli):
    s = np.zeros(B, dtype=SAMPLING_DTYPE)
    s["temperature_milli"] = t_milli
    s["top_k"] = top_k
    s["top_p_milli"] = top_p_milli
    s["session_key"] = np.arange(B, dtype=np.uint64)
    return s


CONFIG_NAMES = ("tiny", "b64", "b256_topk_topp", "ragged", "large")


def make(name: str, device="cpu", sessions: int | None = None, draft_top_n: int = 8,
         chunk_sessions: int = 32, logits: str | None = None) -> Workload:
    """Build a named workload.  ``sessions`` truncates B (same rows as the
    full workload's first sessions), for CPU-sized runs of the big shapes.
    ``logits`` ("bf16" or "fp32") overrides the workload's element type: the
    same draws, stored as binary32 or rounded to bf16."""
    idx = CONFIG_NAMES.index(name)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + idx)
    dev = torch.device(device)

    if name == "tiny":
        B, M, V, dt = 4, 4, 1024, torch.float32
        T, K, P = 1000, 0, 1000
    elif name == "b64":
        B, M, V, dt = 64, 4, 32000, torch.bfloat16
        T, K, P = 1000, 0, 1000
    elif name == "b256_topk_topp":
        B, M, V, dt = 256, 8, 128256, torch.bfloat16
        T, K, P = 700, 50, 900
    elif name == "ragged":
        B, M, V, dt = 512, 16, 151936, torch.bfloat16
        T, K, P = 800, 0, 950
    else:
        B, M, V, dt = 1024, 64, 129280, torch.bfloat16
        T, K, P = 1000, 0, 950
    if logits is not None:
        dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[logits]
    B_full = B
    if sessions is not None:
        B = min(B, sessions)

    # per-session structure, drawn for the full batch so that a truncated
    # workload holds the same first sessions
    if name == "tiny":
        m_full = torch.full((B_full,), M, dtype=torch.int32)
        rule_full = torch.tensor([1, 1, 2, 2], dtype=torch.int32)
    elif name == "ragged":
        g_cpu = torch.Generator().manual_seed(2000 + idx)
        m_full = torch.randint(1, M + 1, (B_full,), generator=g_cpu, dtype=torch.int32)
        kind_perm = torch.randperm(B_full, generator=g_cpu)
        draft_kind_full = torch.empty(B_full, dtype=torch.int64)
        draft_kind_full[kind_perm[: B_full // 4]] = 0  # identical to the target
        draft_kind_full[kind_perm[B_full // 4: 3 * B_full // 4]] = 1  # target + N(0,1)
        draft_kind_full[kind_perm[3 * B_full // 4:]] = 2  # -0.5 * target + N(0,1)
        greedy_perm = torch.randperm(B_full, generator=g_cpu)
        rule_full = torch.full((B_full,), 2, dtype=torch.int32)
        rule_full[greedy_perm[: int(round(0.3 * B_full))]] = 1
    else:
        m_full = torch.full((B_full,), M, dtype=torch.int32)
        rule_full = torch.full((B_full,), 2, dtype=torch.int32)
    m = m_full[:B].clone()
    rule = rule_full[:B].clone()

    target = torch.empty((B, M + 1, V), dtype=dt, device=dev)
    draft = torch.empty((B, M, V), dtype=dt, device=dev)
    tokens = torch.empty((B, M), dtype=torch.int32, device=dev)

    boost_ids = None
    if name == "b64":
        g_cpu = torch.Generator().manual_seed(3000 + idx)
        boost_ids = torch.randperm(V, generator=g_cpu)[: V // 100].to(dev)

    # draw session chunks in order so that any prefix of sessions is identical
    for s0 in range(0, B_full, chunk_sessions):
        if s0 >= B:
            break
        s1 = min(s0 + chunk_sessions, B_full)
        nb = s1 - s0
        if name == "tiny":
            t32 = torch.randn((nb, M + 1, V), generator=gen, device=dev) * 2.0
            d32 = t32[:, :M] + torch.randn((nb, M, V), generator=gen, device=dev) * 0.5
        elif name == "b64":
            t32 = torch.randn((nb, M + 1, V), generator=gen, device=dev) * 3.0
            t32[:, :, boost_ids] += 6.0
            d32 = t32[:, :M] + torch.randn((nb, M, V), generator=gen, device=dev) * 1.0
        elif name == "b256_topk_topp":
            t32 = torch.randn((nb, M + 1, V), generator=gen, device=dev) * 2.0
            heavy = torch.rand((nb, M + 1, V), generator=gen, device=dev) < 0.005
            t32 += heavy.float() * 8.0
            d32 = 0.8 * t32[:, :M] + torch.randn((nb, M, V), generator=gen, device=dev) * 1.5
        elif name == "ragged":
            t32 = torch.randn((nb, M + 1, V), generator=gen, device=dev) * 2.0
            noise = torch.randn((nb, M, V), generator=gen, device=dev)
            kind = draft_kind_full[s0:s1].to(dev).view(nb, 1, 1)
            d32 = torch.where(kind == 0, t32[:, :M],
                              torch.where(kind == 1, t32[:, :M] + noise,
                                          -0.5 * t32[:, :M] + noise))
        else:  # large
            t32 = torch.randn((nb, M + 1, V), generator=gen, device=dev) * 2.5
            peak = torch.randint(0, V, (nb, M + 1, 1), generator=gen, device=dev)
            t32.scatter_add_(2, peak, torch.full((nb, M + 1, 1), 10.0, device=dev))
            d32 = t32[:, :M] + torch.randn((nb, M, V), generator=gen, device=dev) * 2.0
        tq = _to_storage(t32, dt)
        dq = _to_storage(d32, dt)
        hi = min(s1, B)
        target[s0:hi] = tq[: hi - s0]
        draft[s0:hi] = dq[: hi - s0]

        # draft tokens
        untruncated = (K == 0 and P >= 1000)
        top_n = None if untruncated else draft_top_n
        picks = _gumbel_pick(dq.float(), T / 1000.0, gen, top_n)  # [nb, M]
        if name == "ragged":
            greedy = (rule_full[s0:s1] == 1).to(dev).view(nb, 1)
            picks = torch.where(greedy, torch.argmax(dq.float(), dim=-1).to(torch.int32), picks)
        tokens[s0:hi] = picks[: hi - s0]
        del t32, d32, tq, dq

    sampling = _sampling(B, T, K, P)
    return Workload(name=name, target=target, draft=draft, tokens=tokens,
                    m=m.to(dev), rule=rule.to(dev), sampling=sampling, seed=0, round=1)


def to_numpy(w: Workload, sessions=None):
    """Host copies (bf16 as uint16 bits) of a workload, optionally a session slice."""
    if sessions is None:
        sl = slice(None)
        sl_np = slice(None)
    else:
        sl_np = np.asarray(torch.as_tensor(sessions).cpu().numpy(), dtype=np.int64)
        sl = torch.as_tensor(sl_np, device=w.target.device)

    def rows(t):
        if t is None:
            return None
        t = t[sl].contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    return dict(
        target=rows(w.target), draft=rows(w.draft),
        tokens=w.tokens[sl].cpu().numpy().astype(np.int32),
        m=w.m[sl].cpu().numpy().astype(np.int32),
        rule=w.rule[sl].cpu().numpy().astype(np.int32),
        sampling=w.sampling[sl_np].copy(), seed=w.seed, round=w.round,
    )


def bytes_human(n: int) -> str:
    units = ["B", "KB", "MB", "GB", "TB"]
    k = min(int(math.log(max(n, 1), 1000)), len(units) - 1)
    return f"{n / 1000 ** k:.3f} {units[k]}"
