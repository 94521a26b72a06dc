"""GPU parity of sv_commit, the verifier's commit step (SDCP Sec. 4.2, Sec.
6.3 steps 6-8, Sec. 6.5), against the oracle's ov_commit on the same seeded
inputs over many rounds, bit for bit (truncated tokens, committed counts,
actions and every state byte, digests included); and SDCP Appendix A's worked
greedy round through the whole GPU path (sv_verify, then sv_commit)."""
import hashlib
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from tests import parity

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def random_contracts(rng, B):
    c = np.zeros(B, dtype=oracle.CONTRACT_DTYPE)
    c["m_max"] = rng.integers(1, 65, B)
    c["max_new"] = np.where(rng.random(B) < 0.2, rng.integers(0, 40, B), rng.integers(100, 5000, B))
    c["low_rounds"] = rng.integers(1, 5, B)
    c["low_ratio"] = np.where(rng.random(B) < 0.5, 0, rng.integers(1, 101, B))
    c["n_stop"] = rng.integers(0, 11, B)          # above 8: only 8 are used
    c["stop"] = rng.integers(0, 30, (B, 8))
    c["n_fallback"] = rng.integers(0, 11, B)      # above 8: only 8 are used
    c["fallback"] = rng.choice(np.array([1, 2, 3, 5], np.uint8), (B, 8))
    return c


def random_round(rng, B, M):
    a = rng.integers(0, M + 1, B).astype(np.int32)
    a[rng.random(B) < 0.4] = 0                     # many low rounds
    a[rng.random(B) < 0.05] = -3                   # failed sessions
    a[rng.random(B) < 0.02] = M + 1                # out of range: no verdict
    out = np.full((B, M + 1), -1, np.int32)
    for b in range(B):
        if 0 <= a[b] <= M:
            out[b, :a[b] + 1] = rng.integers(0, 400, a[b] + 1)
    m = np.minimum(np.maximum(a, 0) + rng.integers(0, 3, B), M).astype(np.int32)
    m = np.maximum(m, 1)
    return m, a, out


def test_commit_matches_oracle_over_many_rounds():
    import token_sampling_amd as sv
    rng = np.random.default_rng(90)
    B, M = 150, 8  # B not a multiple of the 64 sessions per workgroup
    contracts = random_contracts(rng, B)
    states = np.zeros(B, dtype=oracle.STATE_DTYPE)
    states["digest"] = rng.integers(0, 256, (B, 32), dtype=np.uint8)
    states["m_cap"] = rng.integers(1, 65, B)
    c_dev = torch.from_numpy(contracts.view(np.uint8).reshape(B, 64).copy()).cuda()
    s_dev = torch.from_numpy(states.view(np.uint8).reshape(B, 64).copy()).cuda()
    for r in range(40):
        m, a, out = random_round(rng, B, M)
        ok = (rng.random(B) < 0.5).astype(np.uint8) if r % 2 else None
        parity.log(f"[case] commit round {r}")
        out_dev = torch.from_numpy(out.copy()).cuda()
        res = sv.commit(c_dev, s_dev, torch.from_numpy(m).cuda(), torch.from_numpy(a).cuda(),
                        out_dev, None if ok is None else torch.from_numpy(ok).cuda())
        torch.cuda.synchronize()
        o_out, o_e, o_act = oracle.commit(contracts, states, m, a, out, ok)
        assert np.array_equal(out_dev.cpu().numpy(), o_out), r
        assert np.array_equal(res["emitted_len"].cpu().numpy(), o_e), r
        assert np.array_equal(res["action"].cpu().numpy(), o_act), r
        g_states = sv.states_numpy(s_dev)
        assert g_states.tobytes() == states.tobytes(), r
    acts = set(o_act.tolist())
    parity.log(f"[commit] actions in the last round: {sorted(acts)}, n max {states['n'].max()}")


def test_commit_long_chains_at_m_64():
    """M = 64: up to 65 links per session in one round."""
    import token_sampling_amd as sv
    rng = np.random.default_rng(91)
    B, M = 70, 64
    contracts = oracle.make_contracts(B, m_max=64, max_new=10_000, low_rounds=2, stop=())
    states = oracle.make_states(B, digest=bytes(range(32)), n=5, m_cap=64)
    c_dev = torch.from_numpy(contracts.view(np.uint8).reshape(B, 64).copy()).cuda()
    s_dev = torch.from_numpy(states.view(np.uint8).reshape(B, 64).copy()).cuda()
    a = rng.integers(0, M + 1, B).astype(np.int32)
    a[:3] = M
    out = np.full((B, M + 1), -1, np.int32)
    for b in range(B):
        out[b, :a[b] + 1] = rng.integers(0, 1 << 31, a[b] + 1)
    m = np.full(B, M, np.int32)
    out_dev = torch.from_numpy(out.copy()).cuda()
    res = sv.commit(c_dev, s_dev, torch.from_numpy(m).cuda(), torch.from_numpy(a).cuda(), out_dev)
    torch.cuda.synchronize()
    o_out, o_e, o_act = oracle.commit(contracts, states, m, a, out)
    assert np.array_equal(out_dev.cpu().numpy(), o_out)
    assert np.array_equal(res["emitted_len"].cpu().numpy(), o_e)
    assert sv.states_numpy(s_dev).tobytes() == states.tobytes()
    # the first session's digest against hashlib
    d = bytes(range(32))
    for t in out[0, :M + 1]:
        d = hashlib.sha256(d + struct.pack(">I", int(t))).digest()
    assert bytes(sv.states_numpy(s_dev)["digest"][0]) == d


def test_appendix_a_greedy_round_on_the_gpu():
    """SDCP Appendix A: committed n = 2 (digest d[2]), proposal [7, 9, 11], target
    argmax 7, 9, 13 and then 5.  sv_verify gives a = 2 and the additional
    token 13; sv_commit gives emitted [7, 9, 13], n = 5, action continue, and
    d[5] = the chain from d[2] over 7, 9, 13."""
    import token_sampling_amd as sv
    g = json.load(open(os.path.join(GOLDEN, "sdcp_appendix_a_digests.json")))
    rnd = json.load(open(os.path.join(GOLDEN, "sdcp_appendix_a_greedy_round.json")))
    V, M = 32, 3
    rng = np.random.default_rng(92)
    t = rng.normal(0, 1, size=(1, M + 1, V)).astype(np.float32)
    for i, am in enumerate(rnd["target_argmax"]):
        t[0, i, am] = t[0, i].max() + 3.0
    target = parity.to_device(oracle.bf16_bits(t))
    tokens = torch.tensor([rnd["proposal"]], dtype=torch.int32, device="cuda")
    m = torch.tensor([M], dtype=torch.int32, device="cuda")
    rule = torch.tensor([1], dtype=torch.int32, device="cuda")
    smp = parity.sampling_bytes(oracle.make_sampling(1, 0, 0, 1000))
    out = sv.verify(target, None, tokens, m, rule, smp, 0, 1)
    contracts = sv.make_contracts(1, m_max=8, max_new=256, low_rounds=3, stop=(2,),
                                  fallback=(sv.ACT_REDUCE, sv.ACT_SWITCH, sv.ACT_SELF_DECODE,
                                            sv.ACT_FAIL))
    states = sv.make_states(1, digest=bytes.fromhex(g["d"][2]), n=rnd["committed_n"], m_cap=8)
    res = sv.commit(contracts, states, m, out["accepted_len"], out["out_tokens"])
    torch.cuda.synchronize()
    assert int(out["accepted_len"][0]) == rnd["expected_accepted"]
    assert out["out_tokens"][0].tolist() == rnd["expected_emitted"] + [-1]
    st = sv.states_numpy(states)[0]
    assert int(res["emitted_len"][0]) == 3 and int(st["n"]) == rnd["expected_new_committed"]
    assert int(res["action"][0]) == sv.ACT_CONTINUE and int(st["c"]) == 0
    d = bytes.fromhex(g["d"][2])
    for tok in rnd["expected_emitted"]:
        d = hashlib.sha256(d + struct.pack(">I", tok)).digest()
    assert bytes(st["digest"]) == d
