"""GPU parity of the relaxed rule (private-use rule 192: accept x_i while
p_i(x_i) > 0, then draw the additional token from p_{a+1}) against the oracle,
mixed with the other rules, on the top-k, dense and binary32 cut-row paths, with
Philox and SDCP values, with draft logits and with published q rows, and on
the b256 workload at full size (every session)."""
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


def relaxed_case(seed, B, M, V, dtype):
    h = mixed_case(seed, B, M, V, dtype)
    rng = np.random.default_rng(seed + 700)
    h["rule"] = rng.choice(np.array([1, 2, 192, 192], np.int32), B)
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    # relaxed sessions: proposals from the target's own profile half of the time
    for b in np.nonzero(h["rule"] == 192)[0]:
        s = h["sampling"][b]
        prof = (int(s["temperature_milli"]), int(s["top_k"]), int(s["top_p_milli"]))
        for i in range(M):
            if rng.random() < 0.6:
                st, p, _ = oracle.profile(h["target"][b, i], *prof)
                if st == 0:
                    h["tokens"][b, i] = rng.choice(V, p=p / p.sum())
            else:
                h["tokens"][b, i] = rng.integers(0, V)
    return h


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed,B,M,V", [(101, 28, 6, 2500), (102, 16, 4, 9000)])
def test_relaxed_mixed(dtype, seed, B, M, V):
    parity.log(f"[case] relaxed mixed dtype={dtype} seed={seed} B={B} M={M} V={V}")
    h = relaxed_case(seed, B, M, V, dtype)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    rep = parity.compare(g, o, f"relaxed-{dtype}-{seed}")
    assert (o["accepted_len"][h["rule"] == 192] >= 0).all()
    assert rep["ok_sessions"] > B // 2


def test_relaxed_with_sdcp_values_and_q_rows():
    parity.log("[case] relaxed with SDCP values; with q rows")
    h = relaxed_case(103, 20, 5, 4000, "bf16")
    h["sdcp"] = parity.random_sdcp_sessions(20, np.random.default_rng(11))
    parity.compare(parity.run_gpu(h), parity.run_oracle(h), "relaxed-sdcp")
    # published q rows for the rule-2 sessions; relaxed sessions never read them
    q = np.full((20, 5, 4000), np.nan, np.float32)
    for b in np.nonzero(h["rule"] == 2)[0]:
        s = h["sampling"][b]
        prof = (int(s["temperature_milli"]), int(s["top_k"]), int(s["top_p_milli"]))
        for i in range(5):
            q[b, i] = oracle.profile(h["draft"][b, i], *prof)[1].astype(np.float32)
    h2 = dict(h, draft=None, q_rows=q)
    h2.pop("sdcp")
    parity.compare(parity.run_gpu(h2), parity.run_oracle(h2), "relaxed-qrows")


def test_relaxed_b256_full_size_every_session():
    parity.log("[case] relaxed rule on b256_topk_topp full size, every session")
    w = W.make("b256_topk_topp", device="cuda")
    import token_sampling_amd as sv
    rule = torch.full_like(w.rule, 192)
    out = sv.verify(w.target, None, w.tokens, w.m, rule, w.sampling_tensor("cuda"), w.seed,
                    w.round, probe=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    assert (g["accepted_len"] >= 0).all()
    del out

    def relaxed(ids, h):
        h["draft"] = None
        h["rule"] = np.full(len(ids), 192, np.int32)

    o = parity.run_oracle_sessions(w, extra=relaxed)
    rep = parity.compare(g, o, "relaxed-b256-full")
    assert rep["sessions"] == w.B
    parity.log(f"[workload] relaxed b256: mean accepted {g['accepted_len'].mean():.3f}")
