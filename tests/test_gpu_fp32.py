"""GPU parity of binary32 logits rows on the single-pass kernel: the top-k
class (greedy, temperature 0, 1 <= top_k <= 64) on 32-bit keys and rows with
temperature alone (one pass for the maximum and the normaliser); rows with
top-p or top-k above 64 take the exact profile.  Edge cases use values that
bf16 cannot tell apart (ties only in binary32 or only in bf16), denormals,
signed zeros, NaN payloads of both signs, +inf, -inf masks and an odd
vocabulary so that rows start at every 4-byte alignment.  The B=256, M=8,
V=128256 top-k/top-p workload in binary32 is checked on every session."""
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
