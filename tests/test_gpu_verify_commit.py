"""GPU parity of sv_verify_commit: one round's acceptance step and commit step
in one call (SDCP Sec. 6.3 steps 5-8), whose digest links over the drafted
tokens (Sec. 4.2) are computed beside the row stream.

Each round is run twice on the same inputs and states: sv_verify_commit, and
sv_verify (or sv_verify_sdcp) followed by sv_commit.  Verdicts, truncated
tokens, committed counts, actions and every state byte must agree bit for bit,
and the commit must equal the oracle's ov_commit on the same verdict.  The
contracts stop at drafted tokens and run into max_new, so that the committed
prefix ends at every kind of boundary (inside the drafted tokens, at the
additional token, at zero room)."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu

PROFILES = [(1000, 0, 1000), (700, 50, 900), (0, 0, 1000), (800, 5, 1000), (1000, 0, 800),
            (900, 100, 1000)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def random_contracts(rng, B, V):
    c = np.zeros(B, dtype=oracle.CONTRACT_DTYPE)
    c["m_max"] = rng.integers(1, 65, B)
    c["max_new"] = np.where(rng.random(B) < 0.3, rng.integers(0, 30, B), rng.integers(100, 5000, B))
    c["low_rounds"] = rng.integers(1, 5, B)
    c["low_ratio"] = np.where(rng.random(B) < 0.5, 0, rng.integers(1, 101, B))
    c["n_stop"] = np.where(rng.random(B) < 0.6, rng.integers(1, 11, B), 0)
    c["stop"] = rng.integers(0, V, (B, 8))
    c["n_fallback"] = rng.integers(0, 11, B)
    c["fallback"] = rng.choice(np.array([1, 2, 3, 5], np.uint8), (B, 8))
    return c


def random_states(rng, B):
    s = np.zeros(B, dtype=oracle.STATE_DTYPE)
    s["digest"] = rng.integers(0, 256, (B, 32), dtype=np.uint8)
    s["n"] = rng.integers(0, 20, B)
    s["m_cap"] = rng.integers(1, 65, B)
    return s


def round_case(rng, B, M, V):
    t32 = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    d32 = (0.7 * t32[:, :M] + rng.normal(0, 1.0, size=(B, M, V))).astype(np.float32)
    for b in range(0, B, 3):  # identical drafts: long accepted runs
        d32[b] = t32[b, :M]
    s = oracle.make_sampling(B)
    for b in range(B):
        s[b]["temperature_milli"], s[b]["top_k"], s[b]["top_p_milli"] = PROFILES[b % len(PROFILES)]
    m = rng.integers(1, M + 1, size=B).astype(np.int32)
    h = dict(target=oracle.bf16_bits(t32), draft=oracle.bf16_bits(d32),
             tokens=np.zeros((B, M), np.int32), m=m,
             rule=np.where(rng.random(B) < 0.3, 1, 2).astype(np.int32), sampling=s,
             seed=int(rng.integers(0, 1 << 62)), round=int(rng.integers(1, 1000)))
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    h["m"][rng.random(B) < 0.04] = 0  # limit status: nothing committed
    return h


def both_ways(h, contracts, states, ok, sdcp=None):
    """(combined call, verify then commit, raw verdict tokens): device results as numpy."""
    import token_sampling_amd as sv
    B = len(h["m"])
    dev = lambda a: parity.to_device(a)
    t, d = dev(h["target"]), dev(h["draft"])
    tok, m, rule = dev(np.asarray(h["tokens"], np.int32)), dev(h["m"]), dev(h["rule"])
    smp = parity.sampling_bytes(h["sampling"])
    sess = None if sdcp is None else parity.sdcp_bytes(sdcp)
    c_dev = torch.from_numpy(contracts.view(np.uint8).reshape(B, 64).copy()).cuda()
    s1 = torch.from_numpy(states.view(np.uint8).reshape(B, 64).copy()).cuda()
    s2 = s1.clone()
    ok_dev = None if ok is None else torch.from_numpy(ok).cuda()
    one = sv.verify(t, d, tok, m, rule, smp, h["seed"], h["round"], sdcp_sessions=sess,
                    commit=(c_dev, s1, ok_dev))
    two = sv.verify(t, d, tok, m, rule, smp, h["seed"], h["round"], sdcp_sessions=sess)
    raw = two["out_tokens"].clone()
    res = sv.commit(c_dev, s2, m, two["accepted_len"], two["out_tokens"], ok_dev)
    torch.cuda.synchronize()
    a = {k: v.cpu().numpy() for k, v in one.items()}
    a["states"] = sv.states_numpy(s1)
    b = {"accepted_len": two["accepted_len"].cpu().numpy(),
         "out_tokens": two["out_tokens"].cpu().numpy(),
         "emitted_len": res["emitted_len"].cpu().numpy(), "action": res["action"].cpu().numpy(),
         "states": sv.states_numpy(s2)}
    return a, b, raw.cpu().numpy()


def check_round(a, b, raw, contracts, states, m, ok, label):
    for k in ("accepted_len", "out_tokens", "emitted_len", "action"):
        assert np.array_equal(a[k], b[k]), (label, k)
    assert a["states"].tobytes() == b["states"].tobytes(), label
    o_out, o_e, o_act = oracle.commit(contracts, states, m, b["accepted_len"], raw, ok)
    assert np.array_equal(a["out_tokens"], o_out), label
    assert np.array_equal(a["emitted_len"], o_e), label
    assert np.array_equal(a["action"], o_act), label
    assert a["states"].tobytes() == states.tobytes(), label


def test_verify_commit_over_many_rounds():
    """B = 150 (not a multiple of 64), M = 8, V = 64 (stop tokens are hit
    often), 16 rounds with the state carried, Philox and SDCP values
    alternating, self_decode permission on every other round."""
    rng = np.random.default_rng(300)
    B, M, V = 150, 8, 64
    contracts = random_contracts(rng, B, V)
    states = random_states(rng, B)
    seen = {"inside": 0, "additional": 0, "zero_room": 0}
    for r in range(16):
        parity.log(f"[case] verify_commit round {r}")
        h = round_case(rng, B, M, V)
        sdcp = parity.random_sdcp_sessions(B, rng) if r % 2 else None
        ok = (rng.random(B) < 0.5).astype(np.uint8) if r % 4 >= 2 else None
        a, b, raw = both_ways(h, contracts, states, ok, sdcp)
        acc = b["accepted_len"]
        check_round(a, b, raw, contracts, states, h["m"], ok, f"round {r}")
        e = a["emitted_len"]
        v = acc >= 0
        seen["inside"] += int(((e < acc + 1) & (e > 0) & v).sum())
        seen["additional"] += int(((e == acc + 1) & v).sum())
        seen["zero_room"] += int(((e == 0) & v).sum())
    parity.log(f"[verify_commit] committed prefixes ending: {seen}")
    assert all(n > 0 for n in seen.values()), seen


def test_verify_commit_64_links():
    """M = 64 with drafts equal to the targets (every position accepted): up to
    64 links chained beside the rows, one more after the verdict."""
    rng = np.random.default_rng(301)
    B, M, V = 70, 64, 512
    t32 = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    s = oracle.make_sampling(B, 900, 20, 1000)
    h = dict(target=oracle.bf16_bits(t32), draft=oracle.bf16_bits(t32[:, :M]),
             tokens=np.zeros((B, M), np.int32), m=np.full(B, M, np.int32),
             rule=np.full(B, 2, np.int32), sampling=s, seed=5, round=9)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    contracts = oracle.make_contracts(B, m_max=64, max_new=10_000, low_rounds=2, stop=())
    contracts["max_new"][::5] = rng.integers(1, 70, len(contracts[::5]))
    states = random_states(rng, B)
    parity.log("[case] verify_commit M=64")
    a, b, raw = both_ways(h, contracts, states, None)
    assert (b["accepted_len"] == M).sum() > B // 2
    check_round(a, b, raw, contracts, states, h["m"], None, "M=64")


@pytest.mark.parametrize("name", ["b256_topk_topp", "ragged"])
def test_verify_commit_workload_full_size(name):
    """The workloads at full size, in the launch configuration the benchmark
    times: stop tokens at drafted tokens of a third of the sessions, small
    max_new for a fifth."""
    import token_sampling_amd as sv
    parity.log(f"[case] verify_commit {name} full size")
    w = W.make(name, device="cuda")
    B, M = w.B, w.M
    rng = np.random.default_rng(302)
    contracts = random_contracts(rng, B, w.V)
    toks = w.tokens.cpu().numpy()
    mm = w.m.cpu().numpy()
    for b in range(0, B, 3):
        j = int(rng.integers(0, mm[b]))
        contracts["n_stop"][b] = 2
        contracts["stop"][b, 0] = toks[b, j]
    states = random_states(rng, B)
    c_dev = torch.from_numpy(contracts.view(np.uint8).reshape(B, 64).copy()).cuda()
    s1 = torch.from_numpy(states.view(np.uint8).reshape(B, 64).copy()).cuda()
    s2 = s1.clone()
    smp = w.sampling_tensor("cuda")
    one = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, smp, w.seed, w.round,
                    commit=(c_dev, s1, None))
    two = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, smp, w.seed, w.round)
    raw = two["out_tokens"].clone()
    res = sv.commit(c_dev, s2, w.m, two["accepted_len"], two["out_tokens"])
    torch.cuda.synchronize()
    a = {k: v.cpu().numpy() for k, v in one.items()}
    a["states"] = sv.states_numpy(s1)
    b = {"accepted_len": two["accepted_len"].cpu().numpy(),
         "out_tokens": two["out_tokens"].cpu().numpy(),
         "emitted_len": res["emitted_len"].cpu().numpy(), "action": res["action"].cpu().numpy(),
         "states": sv.states_numpy(s2)}
    check_round(a, b, raw.cpu().numpy(), contracts, states, mm, None, name)
    parity.log(f"[verify_commit] {name}: emitted {int(a['emitted_len'].sum())} tokens, "
               f"finished {int((a['action'] == sv.ACT_FINISH).sum())} sessions")
