"""Distribution-level pins for the oracle's speculative-sampling rule.

SDCP Sec. 6.4 (Rule 2) and the textbook's "The acceptance rule" state that,
with draft tokens drawn from q, the emitted tokens follow the target
distribution p exactly.  With target rows that do not depend on the prefix,
the token emitted at output position j (given that position j is reached)
must follow p_j.  The acceptance probability at position i is
alpha_i = sum_y min(p_i(y), q_i(y)), and the expected number of committed
tokens per round is sum_{k=0}^{m} prod_{i<=k} alpha_i, which for a constant
alpha is (1 - alpha^(m+1)) / (1 - alpha) (SDCP Sec. 6.2; the textbook's
"Expected speedup versus acceptance rate" works it out as 3.36 for
alpha = 0.8, k = 4).

Draft tokens are drawn from q (as computed by the oracle) by numpy's
generator, which is independent of the verifier's Philox stream.
"""
import numpy as np
import pytest
from scipy import stats

N_TRIALS = 100_000
SIG = 1e-3


def run_trials(ora, target_rows, draft_rows, prof, n, rng, seed=0):
    """target_rows [M+1, V], draft_rows [M, V] float32; returns oracle output."""
    M1, V = target_rows.shape
    M = M1 - 1
    qs = []
    for i in range(M):
        st, q, _ = ora.profile(draft_rows[i], *prof)
        assert st == 0
        qs.append(q)
    tokens = np.stack([rng.choice(V, size=n, p=q / q.sum()) for q in qs], axis=1).astype(np.int32)
    target = np.broadcast_to(target_rows, (n, M + 1, V)).copy()
    draft = np.broadcast_to(draft_rows, (n, M, V)).copy()
    sampling = ora.make_sampling(n, *prof)
    out = ora.verify(target, draft, tokens, [M] * n, [2] * n, sampling, seed, 1, diagnostics=False)
    return out, qs


def chisq_pvalue(counts, probs):
    n = counts.sum()
    support = probs > 0
    assert counts[~support].sum() == 0, "a token outside the support of p was emitted"
    exp = probs[support] * n / probs[support].sum()
    obs = counts[support]
    # merge bins with small expectations into one
    small = exp < 5
    if small.any():
        exp = np.append(exp[~small], exp[small].sum())
        obs = np.append(obs[~small], obs[small].sum())
    if len(exp) < 2:
        return 1.0
    return stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue


PROFILES = [(1000, 0, 1000), (700, 5, 1000), (1000, 0, 800), (500, 4, 900)]


@pytest.mark.parametrize("prof", PROFILES)
def test_emitted_tokens_follow_the_target_profile(ora, prof):
    rng = np.random.default_rng(100 + PROFILES.index(prof))
    V, M = 12, 3
    target_rows = rng.normal(0, 1.5, size=(M + 1, V)).astype(np.float32)
    draft_rows = (0.6 * target_rows[:M] + rng.normal(0, 1.2, size=(M, V))).astype(np.float32)
    out, _ = run_trials(ora, target_rows, draft_rows, prof, N_TRIALS, rng)
    a = out["accepted_len"]
    assert np.all(a >= 0)
    for j in range(1, M + 2):
        reached = a >= j - 1
        toks = out["out_tokens"][reached, j - 1]
        _, p, _ = ora.profile(target_rows[j - 1], *prof)
        counts = np.bincount(toks, minlength=V)
        pv = chisq_pvalue(counts, p)
        assert pv > SIG, f"position {j}: chi-square p-value {pv}"


def test_acceptance_rate_per_position_is_overlap_mass(ora):
    rng = np.random.default_rng(200)
    V, M = 10, 4
    prof = (900, 0, 1000)
    target_rows = rng.normal(0, 1.0, size=(M + 1, V)).astype(np.float32)
    draft_rows = (target_rows[:M] + rng.normal(0, 1.0, size=(M, V))).astype(np.float32)
    out, qs = run_trials(ora, target_rows, draft_rows, prof, N_TRIALS, rng, seed=5)
    a = out["accepted_len"]
    for i in range(1, M + 1):
        _, p, _ = ora.profile(target_rows[i - 1], *prof)
        alpha = np.minimum(p, qs[i - 1]).sum()
        reached = (a >= i - 1).sum()
        accepted = (a >= i).sum()
        sd = np.sqrt(alpha * (1 - alpha) / reached)
        assert abs(accepted / reached - alpha) < 5 * sd


def test_expected_tokens_per_round_closed_form(ora):
    """alpha = 0.8 at every position, m = 4: (1 - 0.8^5) / 0.2 = 3.3616."""
    rng = np.random.default_rng(300)
    M = 4
    # p = (0.6, 0.4), q = (0.8, 0.2): sum_y min(p, q) = 0.6 + 0.2 = 0.8
    target_rows = np.tile(np.log(np.array([0.6, 0.4], np.float32)), (M + 1, 1)).astype(np.float32)
    draft_rows = np.tile(np.log(np.array([0.8, 0.2], np.float32)), (M, 1)).astype(np.float32)
    out, qs = run_trials(ora, target_rows, draft_rows, (1000, 0, 1000), N_TRIALS, rng, seed=9)
    _, p, _ = ora.profile(target_rows[0], 1000, 0, 1000)
    alpha = np.minimum(p, qs[0]).sum()
    assert abs(alpha - 0.8) < 1e-6
    closed = (1 - alpha ** (M + 1)) / (1 - alpha)
    assert abs(closed - 3.3616) < 1e-5
    committed = out["accepted_len"] + 1
    probs = np.array([alpha ** k * (1 - alpha) for k in range(M)] + [alpha ** M])
    var = (np.arange(1, M + 2) ** 2 * probs).sum() - closed ** 2
    assert abs(committed.mean() - closed) < 5 * np.sqrt(var / N_TRIALS)
    # the committed-length distribution is the truncated geometric one
    counts = np.bincount(committed, minlength=M + 2)[1:]
    assert stats.chisquare(counts, probs * N_TRIALS).pvalue > SIG
