"""GPU parity of sv_verify_sdcp: the verifier values of SDCP Sec. 6.4
(HMAC-SHA-256 keyed by each session's seed, over its id, round, position and
purpose) in place of Philox, against the oracle run with the same per-session
records, to the same bar as the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from tests.test_gpu_parity import mixed_case
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed,B,M,V", [(61, 30, 7, 3000), (62, 17, 3, 12000)])
def test_sdcp_mixed_profiles(dtype, seed, B, M, V):
    parity.log(f"[case] sdcp mixed dtype={dtype} seed={seed} B={B} M={M} V={V}")
    h = mixed_case(seed, B, M, V, dtype)
    h["sdcp"] = parity.random_sdcp_sessions(B, np.random.default_rng(seed + 1000))
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    parity.compare(g, o, f"sdcp-mixed-{dtype}-{seed}")
    # the Philox path on the same rows takes other decisions somewhere
    p = parity.run_oracle({k: v for k, v in h.items() if k != "sdcp"}, diagnostics=False)
    assert not np.array_equal(p["out_tokens"], o["out_tokens"])


def test_sdcp_full_speculation_length():
    """m = 64 with an identical draft: every position accepted, then the
    additional token from the bonus row with the purpose-1 value of position 65."""
    parity.log("[case] sdcp M=64")
    h = mixed_case(63, 6, 64, 500)
    h["m"] = np.array([64, 64, 1, 40, 64, 2], np.int32)
    h["rule"] = np.array([2, 2, 2, 2, 1, 2], np.int32)
    h["tokens"] = parity.draw_valid_tokens(h, np.random.default_rng(4))
    h["draft"] = h["draft"].copy()
    h["draft"][0] = h["target"][0, :64]
    h["tokens"] = parity.draw_valid_tokens(h, np.random.default_rng(5))
    h["sdcp"] = parity.random_sdcp_sessions(6, np.random.default_rng(6))
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    assert o["accepted_len"][0] == 64
    parity.compare(g, o, "sdcp-m64")


def test_sdcp_ignores_seed_round_and_session_key():
    """The SDCP values depend on the session records only: the call's seed and
    round and sampling.session_key do not change the result."""
    parity.log("[case] sdcp ignores the Philox inputs")
    h = mixed_case(64, 12, 5, 2000)
    h["sdcp"] = parity.random_sdcp_sessions(12, np.random.default_rng(7))
    g1 = parity.run_gpu(h)
    h2 = dict(h, seed=h["seed"] ^ 0x5555, round=h["round"] + 9)
    h2["sampling"] = h["sampling"].copy()
    h2["sampling"]["session_key"] += np.uint64(1000)
    g2 = parity.run_gpu(h2)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
    parity.compare(g1, parity.run_oracle(h), "sdcp-ignores")


def test_sdcp_batch_invariant_and_round_sensitive():
    parity.log("[case] sdcp batch invariance and rounds")
    h = mixed_case(65, 10, 6, 3000)
    h["sdcp"] = parity.random_sdcp_sessions(10, np.random.default_rng(8))
    g = parity.run_gpu(h)
    for b in (0, 4, 9):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in h.items()}
        g1 = parity.run_gpu(one)
        for k in g1:
            assert np.array_equal(g1[k][0], g[k][b]), (b, k)
    # the next round of the same sessions: compared with the oracle again
    h3 = dict(h)
    h3["sdcp"] = h["sdcp"].copy()
    h3["sdcp"]["round"] += np.uint32(1)
    g3 = parity.run_gpu(h3)
    parity.compare(g3, parity.run_oracle(h3), "sdcp-next-round")
    assert not np.array_equal(g3["out_tokens"], g["out_tokens"])


def test_sdcp_appendix_a_session_shape():
    """Session records built as in SDCP Appendix A's example (a 16-octet id,
    seed 42 in the profile, round 1) on a small speculative batch."""
    parity.log("[case] sdcp appendix-A-shaped records")
    h = mixed_case(66, 8, 4, 1500)
    h["rule"][:] = 2
    h["tokens"] = parity.draw_valid_tokens(h, np.random.default_rng(9))
    ids = np.zeros((8, 16), np.uint8)
    ids[:, 15] = np.arange(8)
    ids[:, 0] = 0xA5
    h["sdcp"] = oracle.make_sdcp_sessions(8, seed=42, round_=1, ids=ids)
    parity.compare(parity.run_gpu(h), parity.run_oracle(h), "sdcp-appendix-shape")


def test_sdcp_workload_full_size_every_session():
    """The b256 top-k/top-p workload at full size through sv_verify_sdcp in the
    benchmark's launch configuration, every session against the oracle."""
    parity.log("[case] sdcp workload b256_topk_topp full size, every session")
    w = W.make("b256_topk_topp", device="cuda")
    import token_sampling_amd as sv
    recs = parity.random_sdcp_sessions(w.B, np.random.default_rng(10))
    out = sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, w.sampling_tensor("cuda"),
                    w.seed, w.round, probe=True, sdcp_sessions=parity.sdcp_bytes(recs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    a = g["accepted_len"]
    assert np.all((a >= 0) | (a == oracle.S_BAD_PROPOSAL))
    del out

    def with_sdcp(ids, h):
        h["sdcp"] = recs[ids]

    o = parity.run_oracle_sessions(w, extra=with_sdcp)
    rep = parity.compare(g, o, "sdcp-b256-full")
    assert rep["sessions"] == w.B
