"""GPU parity of the draw from rows without a listed support (textbook "The
acceptance rule", SDCP Sec. 6.4 Rule 2): the row cut into 2048-id groups
over several workgroups per session, whose records hold each group's weight
with the cut keys' ties kept and left out; the last workgroup ranks the ties
only in the groups holding a cut.  Cases: heavy ties of both rows' cut keys
across groups and workgroups (aligned and unaligned rows), published q
entries that are unusable at kept and at left-out ties, and a vocabulary of
more groups than the pick stages in LDS."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def tied_case(seed, B, M, V):
    """Integer-valued logits (a handful of levels), so that every cut key has
    hundreds of ties spread over all groups; the drafts differ from the
    targets, so that most sessions reject and draw from the residual."""
    rng = np.random.default_rng(seed)
    t = rng.integers(0, 7, size=(B, M + 1, V)).astype(np.float32) * 0.75
    d = rng.integers(0, 7, size=(B, M, V)).astype(np.float32) * 0.75
    s = oracle.make_sampling(B, 1000, 0, 1000)
    profiles = [(1000, 0, 600), (800, 3000, 1000), (1200, 0, 300), (1000, 25000, 900),
                (700, 0, 990), (1000, 0, 1000)]
    for b in range(B):
        s[b]["temperature_milli"], s[b]["top_k"], s[b]["top_p_milli"] = profiles[b % len(profiles)]
    h = dict(target=oracle.bf16_bits(t), draft=oracle.bf16_bits(d), tokens=np.zeros((B, M), np.int32),
             m=np.full(B, M, np.int32), rule=np.full(B, 2, np.int32), sampling=s,
             seed=int(rng.integers(0, 1 << 62)), round=int(rng.integers(1, 100)))
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    return h


@pytest.mark.parametrize("V", [40_000, 40_003])
@pytest.mark.parametrize("seed", [1, 2])
def test_ties_of_both_cuts_across_groups(seed, V):
    """20 groups per row, 5 workgroups per session: the groups holding p's and
    q's cut differ from session to session; V = 40003 makes rows unaligned."""
    parity.log(f"[case] draw ties across groups seed={seed} V={V}")
    B, M = 12, 3
    h = tied_case(100 + seed, B, M, V)
    o = parity.run_oracle(h)
    a = o["accepted_len"]
    assert ((a >= 0) & (a < M)).sum() >= 4, "enough residual draws"
    parity.compare(parity.run_gpu(h), o, f"draw-ties-{seed}-{V}")


def test_published_q_unusable_at_kept_and_left_out_ties():
    """Position 1 always rejects (p_1(x_1) = 0), so the residual reads q_1
    where p_1 > 0.  p_1 is cut by top-p inside a tied key.  An unusable q entry
    at a left-out tie is never read; one at a kept tie fails the session."""
    parity.log("[case] draw published q at ties")
    B, M, V = 4, 2, 20_000
    rng = np.random.default_rng(77)
    t = rng.integers(0, 5, size=(B, M + 1, V)).astype(np.float32) * 0.5
    s = oracle.make_sampling(B, 1000, 0, 700)
    q = rng.random((B, M, V)).astype(np.float32)
    q /= q.sum(axis=-1, keepdims=True)
    tokens = np.zeros((B, M), np.int32)
    for b in range(B):
        for i in range(M):
            w = q[b, i].astype(np.float64)
            tokens[b, i] = rng.choice(V, p=w / w.sum())
        t[b, 0, tokens[b, 0]] = -np.inf
    tb = oracle.bf16_bits(t)
    for b in range(B):
        st, p, _ = oracle.profile(tb[b, 0], 1000, 0, 700)
        assert st == 0
        vals = oracle.bf16_to_float(tb[b, 0])
        kc = vals[p > 0].min()
        tied = np.nonzero(vals == kc)[0]
        kept = [y for y in tied if p[y] > 0]
        dropped = [y for y in tied if p[y] == 0]
        assert kept and dropped, "the cut must split a tied key"
        if b == 0:
            q[b, 0, dropped[len(dropped) // 2]] = np.nan   # left out: never read
        elif b == 1:
            q[b, 0, kept[len(kept) // 2]] = np.nan         # kept: bad proposal
        elif b == 2:
            q[b, 0, dropped[-1]] = -1.0                    # left out: never read
            q[b, 0, kept[0]] = np.inf                      # kept: bad proposal
    h = dict(target=tb, draft=None, q_rows=q, tokens=tokens, m=np.full(B, M, np.int32),
             rule=np.full(B, 2, np.int32), sampling=s, seed=5, round=6)
    o = parity.run_oracle(h)
    assert list(np.nonzero(o["accepted_len"] == oracle.S_BAD_PROPOSAL)[0]) == [1, 2]
    assert (o["accepted_len"][[0, 3]] == 0).all()
    parity.compare(parity.run_gpu(h), o, "draw-qrows-ties")


def test_more_groups_than_staged():
    """V = 1,100,003: 538 groups per row, more than the pick stages in LDS (512),
    so the pick reads the records where the workgroups stored them; the rows
    are unaligned.  An untruncated session, a tied top-p session and a top-k
    session drawing from whole rows."""
    parity.log("[case] draw with 538 groups per row")
    B, M, V = 3, 1, 1_100_003
    rng = np.random.default_rng(78)
    t = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    t[1] = np.round(t[1] * 2) / 2                      # ties
    d = (t[:, :M] + rng.normal(0, 1.5, size=(B, M, V))).astype(np.float32)
    s = oracle.make_sampling(B, 1000, 0, 1000)
    s[1]["top_p_milli"] = 800
    s[2]["top_k"] = 4000
    h = dict(target=oracle.bf16_bits(t), draft=oracle.bf16_bits(d), tokens=np.zeros((B, M), np.int32),
             m=np.full(B, M, np.int32), rule=np.full(B, 2, np.int32), sampling=s, seed=11, round=12)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    o = parity.run_oracle(h)
    parity.compare(parity.run_gpu(h), o, "draw-1.1M")


def _key_bits(k):
    """bf16 bits of the keys k (key order = value order, +0 at 0x8000)."""
    k = np.asarray(k, np.int64)
    return np.where(k >= 0x8000, k - 0x8000, 0x8000 | (0x8000 - k)).astype(np.uint16)


def _span_row(rng, V, k0, n, ties):
    """One id at each of the n keys k0 .. k0+n-1, `ties` more ids at k0, the
    rest -inf (no mass), in a random order."""
    row = np.full(V, 0xFF80, np.uint16)
    ids = rng.permutation(V)
    row[ids[:n]] = _key_bits(k0 + np.arange(n))
    row[ids[n:n + ties]] = _key_bits(k0)
    return row


def _cut_in_ties(rows, T, k0, ties):
    """A top_p (milli) whose cut falls inside the ties at k0 for every row of
    `rows` (same multiset of logits), and the support's span in keys."""
    keys = lambda b: np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b).astype(np.int64)
    for tp in range(999, 0, -1):
        ok = True
        for r in rows:
            st, p, _ = oracle.profile(r, T, 0, tp)
            k = keys(r.astype(np.int64))
            kept_ties = int(((k == k0) & (p > 0)).sum())
            if st != 0 or k[p > 0].min() != k0 or not 0 < kept_ties <= ties:
                ok = False
                break
        if ok:
            return tp, int(keys(rows[0].astype(np.int64)).max() - k0 + 1)
    raise AssertionError("no top_p cuts inside the ties")


@pytest.mark.parametrize("V", [6144, 5003])
def test_key_table_spans(V):
    """Rows cut by rank at a positive key with few distinct member logits take
    their weights from per-row tables of at most 1535 keys.  Sessions: spans
    of 1535 keys (the largest a table holds) and 1536 (one more: weighed as
    before), 300 and 40 keys, a cut at the smallest positive bf16 value, a
    negative cut, and a target row that fits with a draft row that does not.
    Both residual draws (drafts permuted) and draws from p (drafts equal to
    the targets) occur; V = 6144 gives aligned rows of whole groups, V = 5003
    unaligned rows with a partial group."""
    parity.log(f"[case] draw key-table spans V={V}")
    rng = np.random.default_rng(300 + V)
    one = 0x8000 + 0x3F80      # key of 1.0
    cases = [  # (k0 of p, span of p, span of q, drafts equal)
        (one, 1535, 1535, False), (one, 1536, 1536, False), (one - 128, 300, 300, True),
        (one + 192, 40, 40, False), (0x8001, 200, 200, False), (0x8000 - 0x3F80, 300, 300, False),
        (one, 1535, 1536, False), (one + 128, 800, 800, True)]
    B, M, ties = len(cases), 3, 1200
    tgt = np.zeros((B, M + 1, V), np.uint16)
    dft = np.zeros((B, M, V), np.uint16)
    s = oracle.make_sampling(B)
    spans = []
    for b, (k0, n, nq, same) in enumerate(cases):
        vmax = float(oracle.bf16_to_float(_key_bits(k0 + max(n, nq) - 1)))
        T = int(max(1.0, abs(vmax)) * 2000)   # milli: nearly flat weights over the span
        tgt[b] = [_span_row(rng, V, k0, n, ties) for _ in range(M + 1)]
        dft[b] = tgt[b, :M] if same else [_span_row(rng, V, k0, nq, ties) for _ in range(M)]
        tp, span_p = _cut_in_ties(list(tgt[b]) + list(dft[b]), T, k0, ties + 1)
        spans.append(span_p)
        s[b]["temperature_milli"], s[b]["top_p_milli"] = T, tp
    assert spans[0] == 1535 and spans[1] == 1536
    h = dict(target=tgt, draft=dft, tokens=np.zeros((B, M), np.int32), m=np.full(B, M, np.int32),
             rule=np.full(B, 2, np.int32), sampling=s, seed=31, round=32)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    o = parity.run_oracle(h)
    a = o["accepted_len"]
    assert ((a >= 0) & (a < M)).sum() >= 3 and (a == M).sum() >= 2, a
    parity.compare(parity.run_gpu(h), o, f"draw-key-tables-{V}")
