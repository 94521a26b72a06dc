"""GPU parity of sv_verify_qrows: the draft distributions given as SDCP q_rows
(Sec. 5.2, binary32 probability rows) instead of draft logits, against the
oracle's q_rows mode on the same inputs, to the same bar as the other parity
tests.  Covers the listed-support residual (q gathered at the target's listed
support), the whole-row residual of the per-session sampler, the entries the
rule reads and the ones it must ignore, SDCP values, and the b256 and ragged
workloads at full size on every session."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from tests.test_gpu_parity import PROFILES, mixed_case
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    yield


def dirichlet_row(rng, V, zero_frac=0.2):
    q = rng.dirichlet(np.full(V, 0.5))
    q[rng.random(V) < zero_frac] = 0.0
    if q.sum() == 0:
        q[rng.integers(0, V)] = 1.0
    return (q / q.sum()).astype(np.float32)


def qrows_case(seed, B, M, V, dtype):
    """mixed_case's targets and profiles; q rows are the binary32 draft profile
    (a faithful drafter) for two sessions in three and Dirichlet rows with zeros
    (unrelated to any logits) for the rest; x_i ~ q_i."""
    h = mixed_case(seed, B, M, V, dtype)
    rng = np.random.default_rng(seed + 500)
    q = np.zeros((B, M, V), np.float32)
    for b in range(B):
        prof = PROFILES[b % len(PROFILES)]
        for i in range(M):
            if b % 3 == 0:
                q[b, i] = dirichlet_row(rng, V)
            else:
                st, qq, _ = oracle.profile(h["draft"][b, i], *prof)
                q[b, i] = qq.astype(np.float32) if st == 0 else dirichlet_row(rng, V)
            if h["rule"][b] == 2:
                qi = q[b, i].astype(np.float64)
                h["tokens"][b, i] = rng.choice(V, p=qi / qi.sum())
    h["q_rows"] = q
    h["draft"] = None
    return h


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed,B,M,V", [(71, 28, 6, 2500), (72, 14, 3, 9000), (73, 20, 9, 777)])
def test_qrows_mixed_profiles(dtype, seed, B, M, V):
    parity.log(f"[case] qrows mixed dtype={dtype} seed={seed} B={B} M={M} V={V}")
    h = qrows_case(seed, B, M, V, dtype)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    rep = parity.compare(g, o, f"qrows-mixed-{dtype}-{seed}")
    assert rep["ok_sessions"] == B


def test_qrows_entries_read_and_ignored():
    """Position 1's drafted token has p = 0, so position 1 is always rejected
    and its q row becomes the residual's.  Sessions 0-3 have a listed target
    support (top_k = 20), sessions 4-7 an untruncated one (the sampler's pass)."""
    parity.log("[case] qrows unusable entries")
    B, M, V = 8, 3, 3000
    rng = np.random.default_rng(81)
    t = rng.normal(0, 1.5, size=(B, M + 1, V)).astype(np.float32)
    s = oracle.make_sampling(B, 1000, 0, 1000)
    s["top_k"][:4] = 20
    q = np.stack([[dirichlet_row(rng, V, zero_frac=0.0) for _ in range(M)] for _ in range(B)])
    tokens = np.zeros((B, M), np.int32)
    for b in range(B):
        for i in range(M):
            tokens[b, i] = rng.choice(V, p=q[b, i].astype(np.float64) / q[b, i].sum())
        t[b, 0, tokens[b, 0]] = -np.inf  # p_1(x_1) = 0
    lowest = lambda b: int(np.argmin(np.where(np.isfinite(t[b, 0]), t[b, 0], np.inf)))
    q[0, 0, int(np.argmax(t[0, 0]))] = np.nan        # read (p > 0): bad proposal
    q[1, 0, lowest(1)] = np.nan                      # outside the top-20: ignored
    q[2, 1, tokens[2, 1]] = 0.0                      # q(x_2) = 0: bad before any draw
    q[3, 0, tokens[3, 0]] = -1.0                     # q(x_1) < 0: bad before any draw
    q[4, 0, int(np.argmax(t[4, 0]))] = np.nan        # read by the sampler's pass
    dead = int(rng.integers(0, V))
    t[5, 0, dead] = -np.inf
    q[5, 0, dead] = np.inf                           # p = 0 there: ignored
    q[6, 0, 17 if tokens[6, 0] != 17 else 18] = -1e-3  # read (p > 0): bad proposal
    h = dict(target=oracle.bf16_bits(t), draft=None, q_rows=q.astype(np.float32), tokens=tokens,
             m=np.full(B, M, np.int32), rule=np.full(B, 2, np.int32), sampling=s, seed=9, round=4)
    g = parity.run_gpu(h)
    o = parity.run_oracle(h)
    want_bad = [0, 2, 3, 4, 6]
    assert list(np.nonzero(o["accepted_len"] == oracle.S_BAD_PROPOSAL)[0]) == want_bad
    assert (o["accepted_len"][[1, 5, 7]] == 0).all()
    parity.compare(g, o, "qrows-entries")


def test_qrows_no_rows_and_greedy():
    parity.log("[case] qrows absent, and greedy sessions")
    h = qrows_case(82, 10, 4, 1000, "bf16")
    h["rule"] = np.array([1, 2] * 5, np.int32)
    h["tokens"] = parity.draw_valid_tokens(dict(h, draft=None), np.random.default_rng(2))
    h["q_rows"][0::2] = np.nan  # greedy sessions never read their rows
    parity.compare(parity.run_gpu(h), parity.run_oracle(h), "qrows-greedy")
    h2 = dict(h)
    h2.pop("q_rows")
    g = parity.run_gpu(h2)
    o = parity.run_oracle(h2)
    assert (o["accepted_len"][1::2] == oracle.S_Q_UNAVAILABLE).all()
    parity.compare(g, o, "qrows-absent")


def test_qrows_with_sdcp_values():
    parity.log("[case] qrows with SDCP values")
    h = qrows_case(83, 18, 5, 4000, "bf16")
    h["sdcp"] = parity.random_sdcp_sessions(18, np.random.default_rng(3))
    parity.compare(parity.run_gpu(h), parity.run_oracle(h), "qrows-sdcp")


@pytest.mark.parametrize("name", ["b256_topk_topp", "ragged"])
def test_qrows_workload_full_size_every_session(name):
    """The workload's target rows with the synthetic drafter's published rows
    (its top-8 at temperature T, the distribution its tokens were drawn from),
    every session against the oracle."""
    parity.log(f"[case] qrows workload {name} full size, every session")
    w = W.make(name, device="cuda")
    q = w.drafter_q_rows()
    import token_sampling_amd as sv
    out = sv.verify(w.target, None, w.tokens, w.m, w.rule, w.sampling_tensor("cuda"), w.seed,
                    w.round, probe=True, q_rows=q)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    a = g["accepted_len"]
    assert (a >= 0).all()  # every token was drawn from its published row
    del out

    def with_q(ids, h):
        h["draft"] = None
        h["q_rows"] = q[torch.as_tensor(ids, device="cuda")].cpu().numpy()

    o = parity.run_oracle_sessions(w, extra=with_q)
    rep = parity.compare(g, o, f"qrows-{name}-full")
    assert rep["sessions"] == w.B
    parity.log(f"[workload] {name} with q rows: mean accepted {a.mean():.3f}")
