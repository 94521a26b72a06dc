"""GPU parity: the HIP path (through the C ABI) against the oracle, element by
element, on seeded synthetic inputs.

Small cases span many profiles, ragged m, both dtypes, ties, -inf masks and
every per-session status; the workload shapes are checked on every session, in
the same launch configuration the benchmark times (B=1024, M=64: every
verdict against the oracle's in-order reading, probes on 32 sessions).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu

PROFILES = [
    (1000, 0, 1000), (700, 50, 900), (800, 0, 950), (0, 0, 1000), (1300, 7, 1000),
    (500, 0, 0), (1000, 1, 1000), (900, 2000, 1000), (600, 30, 500), (2000, 0, 990),
    (1, 0, 1000), (1000, 100000, 999), (700, 3, 300), (1000, 0, 1),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def mixed_case(seed, B, M, V, dtype="bf16", identical_every=5, mask_every=7):
    rng = np.random.default_rng(seed)
    t32 = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    t32 += (rng.random(t32.shape) < 0.005) * np.float32(8)
    d32 = (0.7 * t32[:, :M] + rng.normal(0, 1.2, size=(B, M, V))).astype(np.float32)
    for b in range(0, B, identical_every):
        d32[b] = t32[b, :M]
    for b in range(3, B, mask_every):  # grammar-style -inf masks
        mask = rng.random(V) < 0.6
        mask[rng.integers(0, V)] = False
        t32[b, :, mask] = -np.inf
        d32[b, :, mask] = -np.inf
    if dtype == "bf16":
        target, draft = oracle.bf16_bits(t32), oracle.bf16_bits(d32)
    else:
        target, draft = t32, d32
    s = oracle.make_sampling(B)
    for b in range(B):
        s[b]["temperature_milli"], s[b]["top_k"], s[b]["top_p_milli"] = PROFILES[b % len(PROFILES)]
    h = dict(target=target, draft=draft, tokens=np.zeros((B, M), np.int32),
             m=rng.integers(1, M + 1, size=B).astype(np.int32),
             rule=np.where(rng.random(B) < 0.3, 1, 2).astype(np.int32),
             sampling=s, seed=int(rng.integers(0, 1 << 62)), round=int(rng.integers(1, 1000)))
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    return h


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed,B,M,V", [(11, 28, 6, 2500), (12, 14, 3, 9000), (13, 20, 9, 777)])
def test_mixed_profiles(dtype, seed, B, M, V):
    parity.log(f"[case] mixed dtype={dtype} seed={seed} B={B} M={M} V={V}")
    h = mixed_case(seed, B, M, V, dtype)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    parity.compare(g, o, f"mixed-{dtype}-{seed}")


def test_edge_cases():
    parity.log("[case] edge cases")
    B, M, V = 16, 4, 300
    rng = np.random.default_rng(21)
    t = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.5, size=(B, M, V))).astype(np.float32)
    s = oracle.make_sampling(B, 1000, 0, 1000)
    m = np.full(B, M, np.int32)
    rule = np.full(B, 2, np.int32)
    # 0: all logits equal (every token tied), top-k 3
    t[0] = 0.0; d[0] = 0.0; s[0]["top_k"] = 3
    # 1: all equal, top-p 0.5
    t[1] = 1.5; d[1] = 1.5; s[1]["top_p_milli"] = 500
    # 2: signed zeros and ties at the top
    t[2] = -1.0; t[2, :, ::2] = -0.0; t[2, :, 1::2] = 0.0; d[2] = t[2, :M]; s[2]["top_k"] = 5
    # 3: only two finite tokens
    t[3] = -np.inf; t[3, :, 7] = 1.0; t[3, :, 200] = 1.0; d[3] = t[3, :M]
    # 4: NaN in a draft row -> bad logits
    d[4, 2, 17] = np.nan
    # 5: +inf in the bonus row
    t[5, M, 3] = np.inf
    # 6: m = 0 and 7: m = M + 1 -> limit
    m[6] = 0; m[7] = M + 1
    # 8: top_p 1001 -> bad profile; 9: reserved != 0; 10: unknown rule
    s[8]["top_p_milli"] = 1001; s[9]["reserved"] = 7; rule[10] = 5
    # 11: greedy with a NaN only in the (unread) draft
    rule[11] = 1; d[11, 0, 0] = np.nan
    # 12: temperature 0 under rule 2
    s[12]["temperature_milli"] = 0
    # 13: top_k 1 and 14: top_p 0 (both one-hot)
    s[13]["top_k"] = 1; s[14]["top_p_milli"] = 0
    # 15: huge temperature (near uniform)
    s[15]["temperature_milli"] = 4_000_000_000
    h = dict(target=oracle.bf16_bits(t), draft=oracle.bf16_bits(d), tokens=np.zeros((B, M), np.int32),
             m=m, rule=rule, sampling=s, seed=5, round=3)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    h["tokens"][12] = np.argmax(oracle.bf16_to_float(h["draft"][12]), axis=-1)
    tok = h["tokens"]
    tok[9, 1] = V  # (also out of range, but the profile check comes first)
    bad = dict(h)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    assert o["accepted_len"][4] == oracle.S_BAD_LOGITS
    assert o["accepted_len"][5] == oracle.S_BAD_LOGITS
    assert o["accepted_len"][6] == o["accepted_len"][7] == oracle.S_LIMIT
    assert o["accepted_len"][8] == o["accepted_len"][9] == o["accepted_len"][10] == oracle.S_BAD_PROFILE
    assert o["accepted_len"][11] >= 0
    parity.compare(g, o, "edge")
    # tokens out of range and q(x) = 0
    bad["tokens"] = h["tokens"].copy()
    bad["tokens"][0, 2] = -3
    bad["tokens"][1, 0] = V
    dd = oracle.bf16_to_float(h["draft"]).copy()
    dd[2, 1, bad["tokens"][2, 1]] = -np.inf
    bad["draft"] = oracle.bf16_bits(dd)
    g = parity.run_gpu(bad)
    o = parity.run_oracle(bad)
    assert o["accepted_len"][0] == o["accepted_len"][1] == o["accepted_len"][2] == oracle.S_BAD_PROPOSAL
    parity.compare(g, o, "edge-bad-proposal")


def test_full_speculation_length_and_tiny_vocab():
    parity.log("[case] M=64 and V=1")
    h = mixed_case(31, 5, 64, 300)
    h["m"] = np.array([64, 1, 33, 64, 17], np.int32)
    h["rule"] = np.array([2, 2, 2, 1, 2], np.int32)
    h["tokens"] = parity.draw_valid_tokens(h, np.random.default_rng(3))
    h["draft"] = oracle.bf16_bits(oracle.bf16_to_float(h["draft"]))
    h["draft"][0] = h["target"][0, :64]  # identical draft: all 64 accepted, then the bonus
    parity.compare(parity.run_gpu(h), parity.run_oracle(h), "m64")
    one = dict(target=np.zeros((2, 2, 1), np.float32), draft=np.zeros((2, 1, 1), np.float32),
               tokens=np.zeros((2, 1), np.int32), m=np.array([1, 1], np.int32),
               rule=np.array([1, 2], np.int32), sampling=oracle.make_sampling(2), seed=0, round=1)
    g = parity.run_gpu(one)
    assert g["accepted_len"].tolist() == [1, 1] and g["out_tokens"].tolist() == [[0, 0], [0, 0]]
    parity.compare(g, parity.run_oracle(one), "V1")


def test_no_draft_rows():
    parity.log("[case] draft = NULL")
    h = mixed_case(41, 10, 4, 1000)
    h["draft"] = None
    h["rule"] = np.array([1, 2] * 5, np.int32)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    assert (o["accepted_len"][1::2] == oracle.S_Q_UNAVAILABLE).all()
    parity.compare(g, o, "no-draft")


def test_deterministic_and_batch_invariant():
    parity.log("[case] determinism and batch invariance")
    h = mixed_case(51, 12, 5, 4000)
    g1 = parity.run_gpu(h)
    g2 = parity.run_gpu(h)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
    for b in (0, 5, 11):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in h.items()}
        g = parity.run_gpu(one)
        for k in g:
            assert np.array_equal(g[k][0], g1[k][b]), (b, k)


@pytest.mark.parametrize("name", ["tiny", "b64"])
def test_workload_in_full(name):
    parity.log(f"[case] workload {name} (all sessions)")
    w = W.make(name, device="cuda")
    h = W.to_numpy(w)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    # b64's rows take the dense path (untruncated): probabilities to 2e-7
    parity.compare(g, o, name, prob_rtol=parity.DENSE_PROB_RTOL)


def _verify_full(w, **kw):
    import token_sampling_amd as sv
    out = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, w.sampling_tensor("cuda"),
                    w.seed, w.round, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name", ["b256_topk_topp", "ragged"])
def test_workload_full_size_every_session(name):
    """The full-size workload in the launch configuration the benchmark times,
    every session checked against the oracle (run unchanged, on blocks of
    sessions over the host's threads)."""
    parity.log(f"[case] workload {name} full size, every session")
    w = W.make(name, device="cuda")
    g = _verify_full(w, probe=True)
    a = g["accepted_len"]
    assert np.all((a >= 0) | (a == oracle.S_BAD_PROPOSAL))
    o = parity.run_oracle_sessions(w)
    # ragged's sampling rows take the dense path (top-p): probabilities to 2e-7
    rep = parity.compare(g, o, f"{name}-full", prob_rtol=parity.DENSE_PROB_RTOL)
    assert rep["sessions"] == w.B
    parity.log(f"[workload] {name}: every session of {w.B} checked, mean accepted "
               f"{a[a >= 0].mean():.3f}, bad proposals {(a == oracle.S_BAD_PROPOSAL).sum()}")


def test_large_every_session():
    """B=1024, M=64: every session's verdict (accepted_len, out_tokens) against
    the oracle's in-order reading, which reads a session's rows only up to the
    position that decides it and, where every row is usable (as here), gives
    the SDCP reading's verdict (pinned by the oracle's own tests); then the
    probes p_i(x_i), q_i(x_i) of sessions 0..31 at every position against the
    oracle's SDCP reading."""
    parity.log("[case] workload large full size, every session's verdict")
    w = W.make("large", device="cuda")
    g = _verify_full(w, probe=True)
    o = parity.run_oracle_sessions(w, early=True)
    verdict = {k: g[k] for k in ("accepted_len", "out_tokens")}
    rep = parity.compare(verdict, o, "large-full-verdicts")
    assert rep["sessions"] == 1024
    idx = np.arange(32)
    o32 = parity.run_oracle_sessions(w, sessions=idx)
    parity.compare({k: v[idx] for k, v in g.items()}, o32, "large-probes-0..31",
                   prob_rtol=parity.DENSE_PROB_RTOL)


def test_topk_kernel_edge_cases():
    """Rows handled by the single-pass top-k path (greedy, T = 0, top_k <= 64),
    with an odd vocabulary so that rows start at every alignment."""
    parity.log("[case] top-k path edge cases, V=4999")
    B, M, V = 16, 3, 4999
    rng = np.random.default_rng(61)
    t = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.7, size=(B, M, V))).astype(np.float32)
    s = oracle.make_sampling(B, 900, 20, 1000)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    t[0] = 1.5; d[0] = 1.5; s[0]["top_k"] = 50                   # every token tied
    t[1] -= 30.0; d[1] -= 30.0; s[1]["top_k"] = 40                # all negative (key mode)
    t[5][:, rng.random(V) < 0.7] = -np.inf                          # -inf masks
    d[5][:, rng.random(V) < 0.7] = -np.inf
    s[5]["top_k"] = 10
    s[6]["temperature_milli"] = 0                                   # T = 0 with max ties
    t[6, :, 100] = t[6].max() + 3; t[6, :, 2000] = t[6, :, 100]
    d[6, :, 50] = d[6].max() + 3; d[6, :, 4000] = d[6, :, 50]
    rule[7] = 1                                                     # greedy, +-0 at the top
    t[7] = -np.abs(t[7]) - 1.0; t[7, :, 333] = -0.0; t[7, :, 444] = 0.0
    s[8]["top_k"] = 64; s[8]["top_p_milli"] = 500
    s[9]["top_k"] = 1
    t[10] = -np.inf; d[10] = -np.inf                                # three finite tokens, k = 5
    for j in (5, 77, 4998):
        t[10, :, j] = rng.normal(); d[10, :, j] = rng.normal()
    s[10]["top_k"] = 5
    s[11]["top_k"] = 64; s[11]["temperature_milli"] = 250
    s[12]["top_k"] = 7; s[12]["top_p_milli"] = 0
    s[13]["top_k"] = 33; s[13]["top_p_milli"] = 990
    # ties at the k-th key: 10 distinct best values, then 150 (session 14) or
    # 40 (session 15) tokens of one value, top_k 20: the final cut resolves
    # them by a search over ids (more than a wave of entries) or by the sort
    for b_, nt in ((14, 150), (15, 40)):
        for r in range(M + 1):
            ids = rng.permutation(V)
            t[b_, r] = rng.normal(0, 1, size=V) - 6.0
            t[b_, r, ids[:10]] = 8.0 + np.arange(10) * 0.25
            t[b_, r, ids[10:10 + nt]] = 5.0
        d[b_] = t[b_, :M]
        s[b_]["top_k"] = 20
    tb, db = oracle.bf16_bits(t), oracle.bf16_bits(d)
    tb[2, 1, 1234] = 0xFFC1          # negative NaN inside a raw-mode row
    tb[3, 0, 17] = 0x7FC3            # positive NaN
    db[4, 2, 4000] = 0x7F80          # +inf in a draft row
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=9, round=4)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    for b in (2, 3, 4):  # tokens of the sessions with bad rows: any in range
        h["tokens"][b] = rng.integers(0, V, size=M)
    h["tokens"][6] = np.argmax(oracle.bf16_to_float(db[6]), axis=-1)
    o = parity.run_oracle(h)
    assert (o["accepted_len"][[2, 3, 4]] == oracle.S_BAD_LOGITS).all()
    g = parity.run_gpu(h)
    parity.compare(g, o, "topk-edges")


@pytest.mark.parametrize("split", ["1", "4", "8"])
def test_dense_kernel_edge_cases(split, monkeypatch):
    """Rows handled by the one-pass dense path (temperature, optional top-p,
    top-k off): a maximum that rises tile after tile, heavy ties at the cut,
    drafted tokens on both sides of a tied cut, a cut below the histogram
    window (the exact fallback), all-negative rows, masks, bad logits; an odd
    vocabulary of five tiles so that rows start at every alignment.  Each row
    by one wave, or split over four (histogram windows and ranks merged)."""
    monkeypatch.setenv("SV_ROWS_SPLIT", split)
    parity.log(f"[case] dense path edge cases, V=5003, split={split}")
    B, M, V = 14, 3, 5003
    rng = np.random.default_rng(73)
    t = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.7, size=(B, M, V))).astype(np.float32)
    s = oracle.make_sampling(B, 1000, 0, 900)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    ramp = np.linspace(-5.0, 20.0, V, dtype=np.float32)             # 0: rising maximum
    t[0] = ramp + rng.normal(0, 0.3, size=(M + 1, V)); d[0] = t[0, :M] + rng.normal(0, 0.3, (M, V))
    t[1] = rng.integers(0, 4, size=(M + 1, V)); d[1] = t[1, :M]     # 1: ties, identical draft
    s[1]["top_p_milli"] = 500
    t[2] = rng.integers(0, 3, size=(M + 1, V)) * 0.5; d[2] = t[2, :M]  # 2, 3: tied cut, chosen x
    t[3] = t[2]; d[3] = d[2]
    s[2]["top_p_milli"] = s[3]["top_p_milli"] = 700
    s[4]["temperature_milli"] = 100_000                              # 4: cut far below the top
    t[5] = -np.abs(t[5]) - 5.0; d[5] = -np.abs(d[5]) - 5.0           # 5: all negative
    s[5]["top_p_milli"] = 800
    t[6][:, rng.random(V) < 0.7] = -np.inf                           # 6: -inf masks
    d[6][:, rng.random(V) < 0.7] = -np.inf
    s[6]["top_p_milli"] = 950
    s[10]["top_p_milli"] = 999; s[10]["temperature_milli"] = 500     # 10: nearly the full row
    s[11]["top_p_milli"] = 1000; s[11]["temperature_milli"] = 250    # 11: untruncated, peaked
    t[11, :, 42] += 12.0; d[11, :, 42] += 12.0
    t[12] = -np.inf; d[12] = -np.inf; t[12, :, 3000] = 1.0; d[12, :, 3000] = 2.0  # 12: one finite
    s[12]["top_p_milli"] = 1000
    s[13]["top_k"] = V; s[13]["top_p_milli"] = 600                   # 13: top_k >= V is off
    t[13] = rng.integers(0, 5, size=(M + 1, V)); d[13] = rng.permutation(t[13, :M].ravel()).reshape(M, V)
    tb, db = oracle.bf16_bits(t), oracle.bf16_bits(d)
    tb[7, 1, 2500] = 0x7FC3          # 7: positive NaN in a target row
    db[8, 2, 17] = 0xFFC1            # 8: negative NaN in a draft row
    tb[9, 3, 4000] = 0x7F80          # 9: +inf in the bonus row
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=13, round=2)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    for b in (7, 8, 9):
        h["tokens"][b] = rng.integers(0, V, size=M)
    # sessions 2 and 3: drafted tokens at a tied cut key (draft == target rows)
    for i in range(M):
        st, p, _ = oracle.profile(tb[2, i], 1000, 0, 700)
        assert st == 0
        ids = np.nonzero(p > 0)[0]
        kc = oracle.bf16_to_float(tb[2, i])[ids].min()            # the cut key's value
        tied = np.nonzero(oracle.bf16_to_float(tb[2, i]) == kc)[0]
        kept = [y for y in tied if p[y] > 0]
        dropped = [y for y in tied if p[y] == 0]
        assert kept and dropped, "the cut must split a tied key"
        h["tokens"][2, i] = kept[-1] if i != 1 else kept[0]   # the last and the first kept tie
        h["tokens"][3, i] = dropped[0]                         # the first tie left out: q(x) = 0
    o = parity.run_oracle(h)
    assert (o["accepted_len"][[7, 8, 9]] == oracle.S_BAD_LOGITS).all()
    assert o["accepted_len"][3] == oracle.S_BAD_PROPOSAL
    assert o["accepted_len"][1] == M                               # identical rows: all accepted
    g = parity.run_gpu(h)
    parity.compare(g, o, "dense-edges")


@pytest.mark.parametrize("split", ["1", "4", "8"])
def test_dense_topk_above_64_edge_cases(split, monkeypatch):
    """Rows with 64 < top_k < V, which the one-pass dense path cuts from its
    histogram window: top-k alone and top-k then top-p, ties split at the
    top-k cut with drafted tokens on both sides of it, all-negative rows, a
    rising maximum, -inf masks leaving fewer than K finite tokens, and a
    window holding fewer than K tokens (the exact fallback)."""
    monkeypatch.setenv("SV_ROWS_SPLIT", split)
    parity.log(f"[case] dense path, top_k above 64, V=5003, split={split}")
    B, M, V = 12, 3, 5003
    rng = np.random.default_rng(74)
    t = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.7, size=(B, M, V))).astype(np.float32)
    s = oracle.make_sampling(B, 1000, 100, 1000)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    s[1]["top_k"] = 65                                                # 1: just above 64
    s[2]["top_k"] = 1000; s[2]["top_p_milli"] = 900                  # 2: top-p inside top-k
    s[3]["top_k"] = 300; s[3]["top_p_milli"] = 999                   # 3: top-p reaches top-k's cut
    t[4] = rng.integers(0, 6, size=(M + 1, V)); d[4] = t[4, :M]      # 4, 5: ties at the top-k cut
    t[5] = t[4]; d[5] = d[4]
    s[4]["top_k"] = s[5]["top_k"] = 1500
    t[6] = -np.abs(t[6]) - 5.0; d[6] = -np.abs(d[6]) - 5.0           # 6: all negative
    s[6]["top_k"] = 200; s[6]["top_p_milli"] = 800
    ramp = np.linspace(-5.0, 20.0, V, dtype=np.float32)              # 7: rising maximum
    t[7] = ramp + rng.normal(0, 0.3, size=(M + 1, V)); d[7] = t[7, :M] + rng.normal(0, 0.3, (M, V))
    s[7]["top_k"] = 400
    t[8][:, rng.random(V) < 0.99] = -np.inf                          # 8: fewer finite than K
    d[8][:, rng.random(V) < 0.99] = -np.inf
    s[8]["top_k"] = 2000
    s[9]["top_k"] = 4000                                             # 9: window < K: fallback
    s[10]["top_k"] = V - 1; s[10]["top_p_milli"] = 950               # 10: V - 1
    s[11]["top_k"] = 129; s[11]["temperature_milli"] = 200           # 11: peaked
    t[11, :, 42] += 6.0; d[11, :, 42] += 6.0
    tb, db = oracle.bf16_bits(t), oracle.bf16_bits(d)
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=14, round=3)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    # sessions 4 and 5: drafted tokens at the tied top-k cut (draft == target rows)
    for i in range(M):
        st, p, _ = oracle.profile(tb[4, i], 1000, 1500, 1000)
        assert st == 0 and (p > 0).sum() == 1500
        vals = oracle.bf16_to_float(tb[4, i])
        ids = np.nonzero(p > 0)[0]
        tied = np.nonzero(vals == vals[ids].min())[0]
        kept = [y for y in tied if p[y] > 0]
        dropped = [y for y in tied if p[y] == 0]
        assert kept and dropped, "the top-k cut must split a tied key"
        h["tokens"][4, i] = kept[-1] if i != 1 else kept[0]
        h["tokens"][5, i] = dropped[0]                            # q(x) = 0: bad proposal
    o = parity.run_oracle(h)
    assert o["accepted_len"][5] == oracle.S_BAD_PROPOSAL
    assert o["accepted_len"][4] == M
    g = parity.run_gpu(h)
    parity.compare(g, o, "dense-topk-edges")


@pytest.mark.parametrize("top_k,top_p", [(100, 1000), (1000, 900), (5000, 950)])
def test_full_size_top_k_above_64(top_k, top_p):
    """The B=256, V=128256 rows under top_k above 64, every session against
    the oracle.  The drafted tokens were drawn under top_k = 50 and top_p =
    0.9; with another cut some fall outside q's support (a bad proposal)."""
    parity.log(f"[case] b256 rows at top_k={top_k} top_p={top_p}, every session")
    w = W.make("b256_topk_topp", device="cuda")
    w.sampling["top_k"] = top_k
    w.sampling["top_p_milli"] = top_p
    g = _verify_full(w, probe=True)
    a = g["accepted_len"]
    assert np.all((a >= 0) | (a == oracle.S_BAD_PROPOSAL))
    o = parity.run_oracle_sessions(w)
    parity.compare(g, o, f"b256-top_k{top_k}-top_p{top_p}")


@pytest.mark.parametrize("split", ["1", "2", "4", "8"])
def test_split_rows_each_factor(split, monkeypatch):
    """The single-pass kernel with each row streamed by 1, 2, 4 or 8 waves
    (forced through SV_ROWS_SPLIT; top-k-class rows use at most 4), on top-k,
    one-hot and dense profiles,
    a vocabulary of one tile (waves with empty parts), and rows that overflow
    the candidate region (profiled exactly by the same wave)."""
    monkeypatch.setenv("SV_ROWS_SPLIT", split)
    parity.log(f"[case] split={split}")
    for seed, B, M, V in ((111, 24, 5, 20000), (112, 12, 3, 300), (113, 8, 2, 4097)):
        h = mixed_case(seed, B, M, V, "bf16")
        if seed == 113:  # ascending logits: many candidates in every part of the row
            ramp = np.linspace(-4, 4, V, dtype=np.float32)
            h["target"][0] = oracle.bf16_bits(np.broadcast_to(ramp, (M + 1, V)))
            h["sampling"][0]["top_k"] = 64
            h["sampling"][0]["temperature_milli"] = 1000
        g = parity.run_gpu(h)
        parity.compare(g, parity.run_oracle(h), f"split{split}-{seed}")
