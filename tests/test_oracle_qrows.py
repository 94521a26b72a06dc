"""Pins for the oracle's q_rows mode (ov_verify_qrows): draft distributions
given as SDCP q_rows (Sec. 5.2, one binary32 probability row per proposed
position) instead of draft logits.

References used: the exactness of speculative sampling for ANY draft
distribution q with tokens drawn from q (SDCP Sec. 6.4, Rule 2; the textbook's
"The acceptance rule"), checked by chi-square on the emitted tokens with q rows
that come from no logits at all; numpy's Philox (independent of the oracle's
generator) and exact rational arithmetic for the decisions of single sessions;
SDCP Sec. 6.3 step 5 for the order of the checks.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

from tests.test_oracle_philox import numpy_block
from tests.test_oracle_stats import chisq_pvalue

SIG = 1e-3


def random_q_rows(rng, M, V, zero_frac=0.3):
    """Dirichlet rows with some exact zeros, stored as binary32."""
    q = rng.dirichlet(np.full(V, 0.7), size=M)
    q[rng.random((M, V)) < zero_frac] = 0.0
    for i in range(M):
        if q[i].sum() == 0:
            q[i, rng.integers(0, V)] = 1.0
    q /= q.sum(axis=1, keepdims=True)
    return q.astype(np.float32)


def draw_from_rows(rng, q_rows, n):
    """[n, M] tokens, column i drawn from q_rows[i] (numpy's generator)."""
    M, V = q_rows.shape
    cols = []
    for i in range(M):
        q = q_rows[i].astype(np.float64)
        cols.append(rng.choice(V, size=n, p=q / q.sum()))
    return np.stack(cols, axis=1).astype(np.int32)


@pytest.mark.parametrize("prof", [(1000, 0, 1000), (700, 4, 1000), (900, 0, 800)])
def test_emitted_tokens_follow_p_for_arbitrary_q_rows(ora, prof):
    """x_i ~ q_i from published rows that share no structure with p: the token
    emitted at each reached position follows p, and the acceptance rate at
    position i is sum_y min(p_i(y), q_i(y))."""
    rng = np.random.default_rng(31 + prof[1])
    V, M, n = 10, 3, 60_000
    target_rows = rng.normal(0, 1.3, size=(M + 1, V)).astype(np.float32)
    q_rows = random_q_rows(rng, M, V).astype(np.float64)
    for i in range(M):  # some overlap with p, so that every position is reached
        q_rows[i, np.argmax(target_rows[i])] += 0.3
    q_rows = (q_rows / q_rows.sum(axis=1, keepdims=True)).astype(np.float32)
    tokens = draw_from_rows(rng, q_rows, n)
    out = ora.verify(np.broadcast_to(target_rows, (n, M + 1, V)).copy(), None, tokens, [M] * n,
                     [2] * n, ora.make_sampling(n, *prof), 4242, 1, diagnostics=False,
                     q_rows=np.broadcast_to(q_rows, (n, M, V)).copy())
    a = out["accepted_len"]
    assert (a >= 0).all()
    ps = [ora.profile(target_rows[j], *prof)[1] for j in range(M + 1)]
    for j in range(M + 1):
        reached = a >= j
        assert reached.sum() > 1000, f"position {j + 1} reached too rarely"
        counts = np.bincount(out["out_tokens"][reached, j], minlength=V)
        assert chisq_pvalue(counts, ps[j]) > SIG, f"position {j + 1}"
    for i in range(M):
        alpha = np.minimum(ps[i], q_rows[i].astype(np.float64)).sum()
        reached = a >= i
        acc = (a[reached] > i).mean()
        se = np.sqrt(alpha * (1 - alpha) / reached.sum())
        assert abs(acc - alpha) < 5 * se + 1e-9, (i, acc, alpha)


def test_decisions_follow_numpy_philox_and_exact_residual(ora):
    """Single sessions recomputed by hand: u_acc(i) from numpy's Philox against
    min(1, p_i(x_i) / q_i(x_i)) with q_i(x_i) the widened binary32 entry, and
    the additional token as the exact rational inverse CDF of
    max(0, p - q) (or p_{m+1}) with u_add(a+1)."""
    rng = np.random.default_rng(77)
    V, M = 7, 3
    checked = 0
    for trial in range(250):
        target = rng.normal(0, 1, size=(1, M + 1, V)).astype(np.float32)
        q_rows = random_q_rows(rng, M, V)[None]
        tokens = draw_from_rows(rng, q_rows[0], 1)
        seed = int(rng.integers(0, 1 << 62))
        skey = int(rng.integers(0, 1 << 62))
        s = ora.make_sampling(1, 800, 0, 1000, session_key=np.array([skey], np.uint64))
        out = ora.verify(target, None, tokens, [M], [2], s, seed, 9, q_rows=q_rows)
        a_want = M
        for i in range(1, M + 1):
            _, p, _ = ora.profile(target[0, i - 1], 800, 0, 1000)
            qx = float(q_rows[0, i - 1, tokens[0, i - 1]])
            u = (numpy_block([9, i, 0, 0], [seed, skey])[0] >> 11) / 2.0**53
            if not Fraction(u) < min(Fraction(1), Fraction(float(p[tokens[0, i - 1]])) / Fraction(qx)):
                a_want = i - 1
                break
        a = int(out["accepted_len"][0])
        if out["d_acc"][0].min() > 1e-12:
            assert a == a_want
        assert np.array_equal(out["out_tokens"][0, :a], tokens[0, :a])
        j = a + 1
        u_add = (numpy_block([9, j, 0, 0], [seed, skey])[1] >> 11) / 2.0**53
        _, p, _ = ora.profile(target[0, j - 1], 800, 0, 1000)
        if a < M:
            q = q_rows[0, j - 1]
            w = [max(Fraction(float(p[y])) - Fraction(float(q[y])), Fraction(0)) if p[y] > 0
                 else Fraction(0) for y in range(V)]
            if sum(w) == 0:
                w = [Fraction(float(v)) for v in p]
        else:
            w = [Fraction(float(v)) for v in p]
        t = Fraction(u_add) * sum(w)
        C, pick = Fraction(0), None
        for y in range(V):
            C += w[y]
            if C > t:
                pick = y
                break
        if out["d_cdf"][0] > 1e-12:
            assert out["out_tokens"][0, a] == pick
            checked += 1
        assert (out["out_tokens"][0, a + 1:] == -1).all()
        # probes: q_tok is the widened entry, p_tok the target profile's value
        for i in range(M):
            assert out["q_tok"][0, i] == float(q_rows[0, i, tokens[0, i]])
    assert checked > 240


@pytest.mark.parametrize("bad", [0.0, -0.25, np.nan, np.inf, -np.inf])
def test_unusable_q_of_proposed_token_is_a_bad_proposal_before_any_draw(ora, bad):
    rng = np.random.default_rng(5)
    V, M = 9, 4
    target = rng.normal(0, 1, size=(1, M + 1, V)).astype(np.float32)
    q_rows = random_q_rows(rng, M, V, zero_frac=0.0)[None]
    tokens = draw_from_rows(rng, q_rows[0], 1)
    q_rows[0, 3, tokens[0, 3]] = bad  # the last position: found before any draw
    for seed in range(20):
        out = ora.verify(target, None, tokens, [M], [2], ora.make_sampling(1), seed, 1,
                         q_rows=q_rows)
        assert out["accepted_len"][0] == -1  # sdcp-bad-proposal
        assert (out["out_tokens"][0] == -1).all()
    # beyond m the row is not read
    out = ora.verify(target, None, tokens, [3], [2], ora.make_sampling(1), 0, 1, q_rows=q_rows)
    assert out["accepted_len"][0] >= 0


def test_residual_reads_q_only_where_p_is_positive(ora):
    """At the first rejection the residual max(0, p - q) reads q(y) only where
    p(y) > 0: an unusable entry there fails the session, one where p(y) = 0 is
    ignored (the result equals that with a zero there)."""
    V, M = 6, 1
    target = np.zeros((1, M + 1, V), np.float32)
    target[0, :, 4:] = -np.inf                     # p = (1/4, 1/4, 1/4, 1/4, 0, 0)
    q = np.array([[[0.0, 0.0, 0.0, 0.0, 0.5, 0.5]]], np.float32)
    q[0, 0, 0] = 0.25                               # x = 0 has q = 1/4 ... p/q = 1
    tokens = np.array([[0]], np.int32)
    # ratio 1: always accepted, the residual never formed -> entries never read
    q_bad = q.copy()
    q_bad[0, 0, 1] = np.nan
    out = ora.verify(target, None, tokens, [1], [2], ora.make_sampling(1), 3, 1, q_rows=q_bad)
    assert out["accepted_len"][0] == 1
    # now x = 0 with q(0) = 0.9: ratio 0.25/0.9, rejected for most seeds
    q2 = np.array([[[0.9, 0.0, 0.0, 0.0, 0.05, 0.05]]], np.float32)
    rejected = 0
    for seed in range(40):
        base = ora.verify(target, None, tokens, [1], [2], ora.make_sampling(1), seed, 1, q_rows=q2)
        if base["accepted_len"][0] == 1:
            continue
        rejected += 1
        # an unusable entry where p(y) = 0 (ids 4, 5) changes nothing
        for v in (np.nan, -3.0, np.inf):
            qq = q2.copy()
            qq[0, 0, 5] = v
            o = ora.verify(target, None, tokens, [1], [2], ora.make_sampling(1), seed, 1, q_rows=qq)
            assert o["accepted_len"][0] == base["accepted_len"][0]
            assert np.array_equal(o["out_tokens"], base["out_tokens"])
        # an unusable entry where p(y) > 0 fails the session
        for v in (np.nan, -1e-3, np.inf):
            qq = q2.copy()
            qq[0, 0, 2] = v
            o = ora.verify(target, None, tokens, [1], [2], ora.make_sampling(1), seed, 1, q_rows=qq)
            assert o["accepted_len"][0] == -1 and (o["out_tokens"][0] == -1).all()
    assert rejected > 20


def test_greedy_sessions_ignore_q_rows_and_missing_rows_are_unavailable(ora):
    rng = np.random.default_rng(9)
    V, M, B = 12, 3, 6
    target = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    tokens = np.argmax(target[:, :M], axis=-1).astype(np.int32)
    q_rows = np.full((B, M, V), np.nan, np.float32)  # never read by rule 1
    out = ora.verify(target, None, tokens, [M] * B, [1] * B, ora.make_sampling(B), 1, 1,
                     q_rows=q_rows)
    assert (out["accepted_len"] == M).all()
    assert np.array_equal(out["out_tokens"][:, :M], tokens)
    out = ora.verify(target, None, tokens, [M] * B, [2] * B, ora.make_sampling(B), 1, 1)
    assert (out["accepted_len"] == -3).all()  # sdcp-q-unavailable


def test_q_rows_of_the_draft_profile_reproduce_the_logits_mode(ora):
    """q rows published as the binary32 rounding of the draft profile give the
    same decisions as the logits mode wherever no decision lies within the
    rounding of q (relative 2^-24) of its threshold."""
    rng = np.random.default_rng(12)
    B, M, V = 40, 4, 50
    target = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    draft = (target[:, :M] + rng.normal(0, 1, size=(B, M, V))).astype(np.float32)
    prof = (900, 20, 950)
    q_rows = np.zeros((B, M, V), np.float32)
    for b in range(B):
        for i in range(M):
            q_rows[b, i] = ora.profile(draft[b, i], *prof)[1].astype(np.float32)
    tokens = np.stack([draw_from_rows(rng, q_rows[b], 1)[0] for b in range(B)]).astype(np.int32)
    s = ora.make_sampling(B, *prof)
    lg = ora.verify(target, draft, tokens, [M] * B, [2] * B, s, 55, 2)
    qr = ora.verify(target, None, tokens, [M] * B, [2] * B, s, 55, 2, q_rows=q_rows)
    same = 0
    for b in range(B):
        if min(lg["d_acc"][b].min(), lg["d_cdf"][b]) < 1e-5:
            continue
        assert lg["accepted_len"][b] == qr["accepted_len"][b], b
        a = lg["accepted_len"][b]
        assert np.array_equal(lg["out_tokens"][b, :a], qr["out_tokens"][b, :a]), b
        if a == M:  # bonus draw does not involve q
            assert lg["out_tokens"][b, a] == qr["out_tokens"][b, a]
        same += 1
    assert same > 30
    np.testing.assert_allclose(qr["q_tok"], lg["q_tok"], rtol=2**-23)
