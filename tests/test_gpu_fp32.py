"""GPU parity of binary32 logits rows: the single-pass kernel's top-k class
(greedy, temperature 0, 1 <= top_k <= 64) on 32-bit keys and rows with
temperature alone (one pass for the maximum and the normaliser), and the
cut-row kernel's rows with top-p or top-k above 64 (a histogram of coarse
keys, then a pass that lists the cut's coarse key; rows it hands back take
the exact profile).  Edge cases use values that bf16 cannot tell apart (ties
only in binary32 or only in bf16), denormals, signed zeros, NaN payloads of
both signs, +inf, -inf masks and an odd vocabulary so that rows start at
every 4-byte alignment.  The B=256, M=8, V=128256 top-k/top-p workload and
the B=512, M=16, V=151936 ragged top-p workload in binary32 are checked on
every session."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def fp32_case(seed, B, M, V):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.7, size=(B, M, V))).astype(np.float32)
    return rng, t, d


def test_fp32_topk_class_edge_cases():
    parity.log("[case] fp32 top-k class edge cases, V=4999")
    B, M, V = 14, 3, 4999
    rng, t, d = fp32_case(91, B, M, V)
    s = oracle.make_sampling(B, 900, 20, 1000)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    t[0] = 1.5; d[0] = 1.5; s[0]["top_k"] = 50                      # every token tied
    t[1] -= 30.0; d[1] -= 30.0; s[1]["top_k"] = 40                   # all negative (key mode)
    # 2: distinct in binary32, tied after rounding to bf16 (1 + k ulp)
    base = np.float32(3.0)
    t[2] = base + rng.integers(0, 40, size=(M + 1, V)).astype(np.float32) * np.float32(2.0 ** -22)
    d[2] = t[2, :M]
    s[2]["top_k"] = 64
    t[3][:, rng.random(V) < 0.7] = -np.inf                             # -inf masks
    d[3][:, rng.random(V) < 0.7] = -np.inf
    s[3]["top_k"] = 10
    s[4]["temperature_milli"] = 0                                      # T = 0 with max ties
    t[4, :, 100] = t[4].max() + 3; t[4, :, 2000] = t[4, :, 100]
    d[4, :, 50] = d[4].max() + 3; d[4, :, 4000] = d[4, :, 50]
    rule[5] = 1                                                        # greedy, +-0 at the top
    t[5] = -np.abs(t[5]) - 1.0; t[5, :, 333] = -0.0; t[5, :, 444] = 0.0
    s[6]["top_k"] = 64; s[6]["top_p_milli"] = 500
    s[7]["top_k"] = 1
    t[8] = -np.inf; d[8] = -np.inf                                     # three finite tokens, k = 5
    for j in (5, 77, 4998):
        t[8, :, j] = rng.normal(); d[8, :, j] = rng.normal()
    s[8]["top_k"] = 5
    # 9: denormals and tiny values at the top of an all-nonpositive row
    t[9] = -np.abs(t[9]) - 1.0; d[9] = -np.abs(d[9]) - 1.0
    t[9, :, 10:20] = np.float32(1e-40); t[9, :, 30] = np.float32(-1e-44)
    d[9, :, 10:20] = np.float32(1e-40)
    s[9]["top_k"] = 16
    s[10]["top_k"] = 33; s[10]["top_p_milli"] = 990
    tb, db = t.copy(), d.copy()
    tb.view(np.uint32)[11, 1, 1234] = 0xFFC00001   # negative NaN inside a raw-mode row
    tb.view(np.uint32)[12, 0, 17] = 0x7FC00003     # positive NaN
    db.view(np.uint32)[13, 2, 4000] = 0x7F800000   # +inf in a draft row
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=19, round=4)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    for b in (11, 12, 13):
        h["tokens"][b] = rng.integers(0, V, size=M)
    h["tokens"][4] = np.argmax(db[4], axis=-1)
    o = parity.run_oracle(h)
    assert (o["accepted_len"][[11, 12, 13]] == oracle.S_BAD_LOGITS).all()
    g = parity.run_gpu(h)
    parity.compare(g, o, "fp32-topk-edges")


def test_fp32_temperature_only_edge_cases():
    parity.log("[case] fp32 rows with temperature alone, V=5003")
    B, M, V = 12, 3, 5003
    rng, t, d = fp32_case(92, B, M, V)
    s = oracle.make_sampling(B, 1000, 0, 1000)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    ramp = np.linspace(-5.0, 60.0, V, dtype=np.float32)              # 0: a rising maximum
    t[0] = ramp + rng.normal(0, 0.3, size=(M + 1, V)); d[0] = t[0, :M] + rng.normal(0, 0.3, (M, V))
    t[1] = rng.integers(0, 4, size=(M + 1, V)); d[1] = t[1, :M]      # 1: ties, identical draft
    s[2]["temperature_milli"] = 250                                   # 2: peaked
    t[2, :, 42] += 12.0; d[2, :, 42] += 12.0
    t[3][:, rng.random(V) < 0.7] = -np.inf                            # 3: -inf masks
    d[3][:, rng.random(V) < 0.7] = -np.inf
    t[4] = -np.inf; d[4] = -np.inf; t[4, :, 3000] = 1.0; d[4, :, 3000] = 2.0  # 4: one finite
    s[5]["temperature_milli"] = 4_000_000_000                         # 5: nearly uniform
    s[6]["temperature_milli"] = 1                                     # 6: T = 0.001
    t[7] *= 40.0; d[7] *= 40.0                                        # 7: wide range
    s[8]["top_k"] = V                                                 # 8: top_k >= V is off
    tb, db = t.copy(), d.copy()
    tb.view(np.uint32)[9, 1, 2500] = 0x7FC00003    # 9: positive NaN in a target row
    db.view(np.uint32)[10, 2, 17] = 0xFFC00001     # 10: negative NaN in a draft row
    tb.view(np.uint32)[11, 3, 4000] = 0x7F800000   # 11: +inf in the bonus row
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=23, round=2)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    for b in (9, 10, 11):
        h["tokens"][b] = rng.integers(0, V, size=M)
    o = parity.run_oracle(h)
    assert (o["accepted_len"][[9, 10, 11]] == oracle.S_BAD_LOGITS).all()
    assert o["accepted_len"][1] == M
    g = parity.run_gpu(h)
    parity.compare(g, o, "fp32-temperature-edges", prob_rtol=parity.DENSE_PROB_RTOL)


def test_fp32_cut_rows_edge_cases():
    """Rows with top-p or top-k above 64: the cut in one coarse key (1/128
    octave) listed and settled on exact keys, top-k and top-p cutting in the
    same or in different coarse keys, ties only in binary32, and the rows the
    kernel hands back to the exact profile (a coarse key with more tokens than
    its list holds, |lmax| / T beyond its precision bound, a cut below the
    window)."""
    parity.log("[case] fp32 cut rows (top-p, top-k above 64), V=5003")
    B, M, V = 18, 3, 5003
    rng, t, d = fp32_case(93, B, M, V)
    s = oracle.make_sampling(B, 800, 0, 900)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    s[1]["top_k"] = 100; s[1]["top_p_milli"] = 1000                     # 1: top-k alone
    s[2]["top_k"] = 200; s[2]["top_p_milli"] = 950                      # 2: both
    s[3]["top_k"] = 70; s[3]["top_p_milli"] = 500                       # 3: both, tighter
    t[4] -= 30.0; d[4] -= 30.0; s[4]["top_p_milli"] = 950               # 4: all negative
    # 5: 600 tokens on 8 binary32 values of one coarse key (ties only in
    # binary32) above a low background, identical draft
    t[5] = rng.normal(-6.0, 1.0, size=(M + 1, V)).astype(np.float32)
    for r in range(M + 1):
        ids = rng.choice(V, size=600, replace=False)
        t[5, r, ids] = np.float32(1.0) + rng.integers(0, 8, size=600).astype(np.float32) * np.float32(2.0 ** -20)
    d[5] = t[5, :M]; s[5]["top_p_milli"] = 700
    # 6: 2000 distinct values in one coarse key: more than the list holds
    t[6] = rng.normal(-8.0, 1.0, size=(M + 1, V)).astype(np.float32)
    for r in range(M + 1):
        ids = rng.choice(V, size=2000, replace=False)
        t[6, r, ids] = np.float32(1.0) + rng.permutation(2000).astype(np.float32) * np.float32(2.0 ** -21)
    d[6] = t[6, :M]; s[6]["top_p_milli"] = 500
    t[7][:, rng.random(V) < 0.7] = -np.inf                              # 7: -inf masks
    d[7][:, rng.random(V) < 0.7] = -np.inf
    t[8] *= 40.0; d[8] *= 40.0; s[8]["temperature_milli"] = 500         # 8: |lmax| / T large
    # 9: denormals and signed zeros of both signs around a few normal values
    t[9] = (rng.normal(0, 1, size=(M + 1, V)) * 1e-39).astype(np.float32)
    t[9, :, ::7] = -0.0; t[9, :, 3::7] = 0.0; t[9, :, 100:110] = 0.5
    d[9] = t[9, :M]; s[9]["temperature_milli"] = 1000
    ramp = np.linspace(-5.0, 30.0, V, dtype=np.float32)               # 10: a rising maximum
    t[10] = ramp + rng.normal(0, 0.3, size=(M + 1, V)); d[10] = t[10, :M] + rng.normal(0, 0.3, (M, V))
    s[10]["top_p_milli"] = 950
    s[11]["top_p_milli"] = 999; s[11]["temperature_milli"] = 3000       # 11: a cut deep down
    s[12]["top_k"] = V - 1; s[12]["top_p_milli"] = 1000                 # 12: top-k just below V
    t[13] = -np.inf; d[13] = -np.inf; t[13, :, 4000] = 1.0; d[13, :, 4000] = 2.0  # 13: one finite
    t[14] = rng.integers(0, 4, size=(M + 1, V)); d[14] = t[14, :M]      # 14: few values, many ties
    s[14]["top_k"] = 300; s[14]["top_p_milli"] = 800
    tb, db = t.copy(), d.copy()
    tb.view(np.uint32)[15, 1, 2500] = 0x7FC00003    # 15: positive NaN
    db.view(np.uint32)[16, 2, 17] = 0xFFC00001      # 16: negative NaN in a draft row
    tb.view(np.uint32)[17, 3, 4000] = 0x7F800000    # 17: +inf in the bonus row
    h = dict(target=tb, draft=db, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=29, round=3)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    for b in (15, 16, 17):
        h["tokens"][b] = rng.integers(0, V, size=M)
    o = parity.run_oracle(h)
    assert (o["accepted_len"][[15, 16, 17]] == oracle.S_BAD_LOGITS).all()
    g = parity.run_gpu(h)
    parity.compare(g, o, "fp32-cut-edges", prob_rtol=parity.DENSE_PROB_RTOL)


@pytest.mark.parametrize("V", [1, 2, 7, 515, 2049, 4096, 4097])
def test_fp32_cut_rows_small_vocabularies(V):
    """Binary32 cut rows on vocabularies of one token up to a few tiles, with
    ties, -inf masks and both signs, under top-p and top-k above 64: up to
    4096 tokens profiled exactly by the single-pass kernel's wave, above by
    the cut-row kernel."""
    parity.log(f"[case] fp32 cut rows, V={V}")
    B, M = 8, 2
    rng, t, d = fp32_case(94 + V, B, M, V)
    s = oracle.make_sampling(B, 1000, 0, 800)
    rule = np.full(B, 2, np.int32)
    m = np.full(B, M, np.int32)
    t[1] = np.round(t[1]); d[1] = t[1, :M]                             # ties
    t[2][:, rng.random(V) < 0.5] = -np.inf; d[2] = t[2, :M]            # masks
    t[3] = -np.abs(t[3]); d[3] = -np.abs(d[3])                          # all negative
    if V > 65:
        s[4]["top_k"] = 65; s[5]["top_k"] = 65; s[5]["top_p_milli"] = 1000
    s[6]["top_p_milli"] = 1; s[7]["temperature_milli"] = 250
    h = dict(target=t, draft=d, tokens=np.zeros((B, M), np.int32), m=m, rule=rule,
             sampling=s, seed=31, round=5)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    o = parity.run_oracle(h)
    g = parity.run_gpu(h)
    parity.compare(g, o, f"fp32-cut-V{V}", prob_rtol=parity.DENSE_PROB_RTOL)


@pytest.mark.parametrize("window", [None, 1])
def test_fp32_ragged_full_size_every_session(window):
    """The B=512, M=16, V=151936 ragged workload (top-p 0.95, 30% greedy
    sessions) with binary32 logits, every session; also read in order
    (windows of positions), where the cut-row kernel takes each window's
    rows."""
    parity.log(f"[case] ragged in fp32, full size, every session, window={window}")
    import token_sampling_amd as sv
    w = W.make("ragged", device="cuda", logits="fp32")
    out = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, w.sampling_tensor("cuda"),
                    w.seed, w.round, probe=True, early=window)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    a = g["accepted_len"]
    assert np.all((a >= 0) | (a == oracle.S_BAD_PROPOSAL))
    del out
    o = parity.run_oracle_sessions(w, early=window is not None)
    rep = parity.compare(g, o, f"fp32-ragged-full-w{window}", prob_rtol=parity.DENSE_PROB_RTOL)
    assert rep["sessions"] == 512


@pytest.mark.parametrize("window", [None, 1])
def test_fp32_b256_full_size_every_session(window):
    """The B=256, M=8, V=128256 top-k 50 / top-p 0.9 workload with binary32
    logits (the same draws, not rounded to bf16), every session."""
    parity.log(f"[case] b256_topk_topp in fp32, full size, every session, window={window}")
    import token_sampling_amd as sv
    w = W.make("b256_topk_topp", device="cuda", logits="fp32")
    out = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, w.sampling_tensor("cuda"),
                    w.seed, w.round, probe=True, early=window)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    a = g["accepted_len"]
    assert np.all((a >= 0) | (a == oracle.S_BAD_PROPOSAL))
    del out
    o = parity.run_oracle_sessions(w, early=window is not None)
    rep = parity.compare(g, o, f"fp32-b256-full-w{window}")
    assert rep["sessions"] == 256
