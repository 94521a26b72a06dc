"""Pins for the oracle's acceptance rules (SDCP Sec. 6.3 step 5 and Sec. 6.4).

References used: the worked greedy round of SDCP Appendix A (golden fixture),
numpy argmax for brute-force greedy prefixes, numpy's Philox (independent of
the oracle's generator) for the uniforms a session must consume, and exact
rational arithmetic for the residual draw.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from tests.test_oracle_philox import numpy_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def batch(ora, target, draft, tokens, m, rule, t=1000, k=0, p=1000, seed=0, rnd=1,
          sampling=None, diagnostics=True):
    B = target.shape[0]
    if sampling is None:
        sampling = ora.make_sampling(B, t, k, p)
    return ora.verify(target, draft, tokens, m, rule, sampling, seed, rnd, diagnostics)


def one_hot_rows(argmaxes, V, rng=None, peak=5.0):
    rows = np.zeros((len(argmaxes), V), dtype=np.float32)
    if rng is not None:
        rows += rng.normal(0, 1, size=rows.shape).astype(np.float32)
    for r, g in enumerate(argmaxes):
        rows[r, g] = rows[r].max() + peak
    return rows


def test_appendix_a_greedy_round(ora):
    fx = json.load(open(os.path.join(GOLDEN, "sdcp_appendix_a_greedy_round.json")))
    M = len(fx["proposal"])
    V = 16
    rng = np.random.default_rng(0)
    target = one_hot_rows(fx["target_argmax"], V, rng)[None]
    draft = rng.normal(0, 1, size=(1, M, V)).astype(np.float32)
    out = batch(ora, target, draft, np.array([fx["proposal"]]), [M], [1])
    a = int(out["accepted_len"][0])
    assert a == fx["expected_accepted"]
    emitted = out["out_tokens"][0, : a + 1].tolist()
    assert emitted == fx["expected_emitted"]
    assert out["out_tokens"][0, a + 1:].tolist() == [-1] * (M - a)
    assert fx["committed_n"] + len(emitted) == fx["expected_new_committed"]
    # SDCP Sec. 6.5.2: with low_ratio absent a round is low iff a = 0
    assert (a == 0) == fx["expected_low"]


def test_greedy_matches_brute_force_prefix(ora):
    rng = np.random.default_rng(1)
    for trial in range(300):
        B, M, V = 3, int(rng.integers(1, 7)), int(rng.integers(2, 9))
        target = np.round(rng.normal(0, 1, size=(B, M + 1, V)) * 2).astype(np.float32)
        draft = rng.normal(0, 1, size=(B, M, V)).astype(np.float32)
        m = rng.integers(1, M + 1, size=B)
        g = np.argmax(target, axis=-1)  # first occurrence = smallest id
        tokens = np.where(rng.random((B, M)) < 0.7, g[:, :M], rng.integers(0, V, (B, M)))
        out = batch(ora, target, draft, tokens, m, [1] * B, seed=int(rng.integers(0, 99)))
        for b in range(B):
            a = 0
            while a < m[b] and tokens[b, a] == g[b, a]:
                a += 1
            assert out["accepted_len"][b] == a
            assert out["out_tokens"][b, :a].tolist() == tokens[b, :a].tolist()
            assert out["out_tokens"][b, a] == g[b, a]
            assert (out["out_tokens"][b, a + 1:] == -1).all()


def test_greedy_ignores_draft_seed_round_and_profile(ora):
    rng = np.random.default_rng(2)
    B, M, V = 4, 5, 12
    target = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    g = np.argmax(target, axis=-1)
    tokens = g[:, :M].copy()
    tokens[1, 2] = (tokens[1, 2] + 1) % V
    ref = batch(ora, target, None, tokens, [M] * B, [1] * B)
    for seed, rnd, t, k, p in [(1, 1, 700, 3, 900), (99, 5, 0, 0, 0), (7, 2, 2000, 1, 1000)]:
        draft = rng.normal(0, 5, size=(B, M, V)).astype(np.float32)
        out = batch(ora, target, draft, tokens, [M] * B, [1] * B, t, k, p, seed, rnd)
        assert np.array_equal(out["accepted_len"], ref["accepted_len"])
        assert np.array_equal(out["out_tokens"], ref["out_tokens"])


def test_identical_draft_accepts_everything(ora):
    rng = np.random.default_rng(3)
    for prof in [(1000, 0, 1000), (700, 5, 900), (300, 0, 500), (1500, 2, 1000)]:
        B, M, V = 16, 6, 40
        target = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
        draft = target[:, :M].copy()
        tokens = np.zeros((B, M), dtype=np.int32)
        for b in range(B):
            for i in range(M):
                _, q, _ = ora.profile(draft[b, i], *prof)
                tokens[b, i] = rng.choice(V, p=q / q.sum())
        m = rng.integers(1, M + 1, size=B)
        out = batch(ora, target, draft, tokens, m, [2] * B, *prof, seed=int(rng.integers(1 << 40)))
        assert np.array_equal(out["accepted_len"], m)
        ratio = out["p_tok"] / out["q_tok"]
        for b in range(B):
            assert np.all(ratio[b, : m[b]] == 1.0)


def test_temperature_zero_speculative_equals_greedy(ora):
    rng = np.random.default_rng(4)
    B, M, V = 40, 5, 10
    target = np.round(rng.normal(0, 1, size=(B, M + 1, V)) * 3).astype(np.float32)
    draft = np.round(rng.normal(0, 1, size=(B, M, V)) * 3).astype(np.float32)
    tokens = np.argmax(draft, axis=-1).astype(np.int32)  # the only valid T=0 proposal
    hit = rng.random((B, M)) < 0.5
    tokens = np.where(hit, np.argmax(target[:, :M], axis=-1), tokens).astype(np.int32)
    draft_fix = draft.copy()
    for b in range(B):
        for i in range(M):
            draft_fix[b, i, tokens[b, i]] = draft_fix[b, i].max() + 1
    m = rng.integers(1, M + 1, size=B)
    spec = batch(ora, target, draft_fix, tokens, m, [2] * B, 0, 0, 1000, seed=3)
    greedy = batch(ora, target, draft_fix, tokens, m, [1] * B)
    assert np.array_equal(spec["accepted_len"], greedy["accepted_len"])
    assert np.array_equal(spec["out_tokens"], greedy["out_tokens"])


def test_emits_between_one_and_m_plus_one(ora):
    rng = np.random.default_rng(5)
    B, M, V = 200, 8, 30
    target = rng.normal(0, 2, size=(B, M + 1, V)).astype(np.float32)
    draft = (target[:, :M] * 0.5 + rng.normal(0, 2, size=(B, M, V))).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, M)).astype(np.int32)
    m = rng.integers(1, M + 1, size=B)
    out = batch(ora, target, draft, tokens, m, [2] * B, 900, 0, 1000, seed=11)
    a = out["accepted_len"]
    assert np.all((a >= 0) & (a <= m))
    n_emit = (out["out_tokens"] >= 0).sum(axis=1)
    assert np.array_equal(n_emit, a + 1)
    assert np.all(out["out_tokens"][out["out_tokens"] >= 0] < V)


def test_zero_target_probability_is_always_rejected(ora):
    rng = np.random.default_rng(6)
    B, M, V = 64, 3, 8
    target = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    draft = rng.normal(0, 1, size=(B, M, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, M)).astype(np.int32)
    for b in range(B):
        target[b, 0, tokens[b, 0]] = -np.inf
    out = batch(ora, target, draft, tokens, [M] * B, [2] * B, seed=5)
    assert np.all(out["accepted_len"] == 0)
    assert np.all(out["out_tokens"][:, 0] != tokens[:, 0])


def test_session_statuses(ora):
    V, M = 6, 3
    rng = np.random.default_rng(7)
    target = rng.normal(0, 1, size=(8, M + 1, V)).astype(np.float32)
    draft = rng.normal(0, 1, size=(8, M, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(8, M)).astype(np.int32)
    m = np.array([0, M + 1, 2, 2, 2, 2, 2, 2])
    rule = np.array([2, 2, 3, 2, 2, 2, 2, 1])
    s = ora.make_sampling(8, 1000, 0, 1000)
    s["top_p_milli"][3] = 1001
    s["reserved"][4] = 1
    tokens[5, 1] = V  # out of range
    draft[6, 1, tokens[6, 1]] = -np.inf  # q(x) = 0
    tokens[7, 0] = -1  # out of range under rule 1 too
    out = ora.verify(target, draft, tokens, m, rule, s, 0, 1)
    assert out["accepted_len"].tolist() == [ora.S_LIMIT, ora.S_LIMIT, ora.S_BAD_PROFILE,
                                            ora.S_BAD_PROFILE, ora.S_BAD_PROFILE,
                                            ora.S_BAD_PROPOSAL, ora.S_BAD_PROPOSAL,
                                            ora.S_BAD_PROPOSAL]
    assert np.all(out["out_tokens"] == -1)
    # no draft rows: rule-2 sessions are q-unavailable, rule-1 sessions run
    out = ora.verify(target[:2], None, np.zeros((2, M), np.int32), [2, 2], [2, 1],
                     ora.make_sampling(2), 0, 1)
    assert out["accepted_len"][0] == ora.S_Q_UNAVAILABLE
    assert out["accepted_len"][1] >= 0


def test_bad_logits_in_any_read_row(ora):
    V, M = 5, 2
    base_t = np.zeros((1, M + 1, V), np.float32)
    base_d = np.zeros((1, M, V), np.float32)
    tok = np.zeros((1, M), np.int32)
    for where, rule in [("t_last", 1), ("t_last", 2), ("d_0", 2)]:
        t, d = base_t.copy(), base_d.copy()
        if where == "t_last":
            t[0, M, 3] = np.nan
        else:
            d[0, 0, :] = -np.inf
        out = ora.verify(t, d, tok, [M], [rule], ora.make_sampling(1), 0, 1)
        assert out["accepted_len"][0] == ora.S_BAD_LOGITS
    # a greedy session never reads draft rows
    d = base_d.copy()
    d[0, 0, 0] = np.nan
    out = ora.verify(base_t, d, tok, [M], [1], ora.make_sampling(1), 0, 1)
    assert out["accepted_len"][0] >= 0


def test_bad_proposal_is_decided_before_any_draw(ora):
    """q(x) = 0 at a later position rejects the round whatever the uniforms."""
    V, M = 4, 3
    target = np.zeros((1, M + 1, V), np.float32)
    draft = np.zeros((1, M, V), np.float32)
    tokens = np.array([[1, 2, 3]], np.int32)
    draft[0, 2, 3] = -np.inf
    for seed in range(50):
        out = ora.verify(target, draft, tokens, [M], [2], ora.make_sampling(1), seed, 1)
        assert out["accepted_len"][0] == ora.S_BAD_PROPOSAL


def test_acceptance_consumes_u_acc_of_position_i(ora):
    """p_i(x_i)/q_i(x_i) = 1/2 exactly: accept iff the numpy-derived u_acc(i) < 1/2."""
    V, M = 2, 4
    target = np.zeros((1, M + 1, V), np.float32)  # p = (1/2, 1/2)
    draft = np.zeros((1, M, V), np.float32)
    draft[0, :, 1] = -np.inf  # q = (1, 0): ratio for x=0 is exactly 1/2
    tokens = np.zeros((1, M), np.int32)
    for seed in range(300):
        skey = 1000 + seed
        s = ora.make_sampling(1, session_key=np.array([skey], np.uint64))
        out = ora.verify(target, draft, tokens, [M], [2], s, seed, 7)
        a = 0
        for i in range(1, M + 1):
            u = (numpy_block([7, i, 0, 0], [seed, skey])[0] >> 11) / 2.0**53
            if u < 0.5:
                a += 1
            else:
                break
        assert out["accepted_len"][0] == a
        # the residual max(0, p - q) is all on token 1 -> the extra token is 1
        if a < M:
            assert out["out_tokens"][0, a] == 1


def test_residual_and_bonus_draws_match_exact_inverse_cdf(ora):
    rng = np.random.default_rng(8)
    V, M = 6, 3
    checked = 0
    for trial in range(200):
        target = rng.normal(0, 1, size=(1, M + 1, V)).astype(np.float32)
        draft = rng.normal(0, 1, size=(1, M, V)).astype(np.float32)
        tokens = rng.integers(0, V, size=(1, M)).astype(np.int32)
        seed = int(rng.integers(0, 1 << 62))
        out = batch(ora, target, draft, tokens, [M], [2], 1000, 0, 1000, seed=seed, rnd=3)
        a = int(out["accepted_len"][0])
        j = a + 1  # position whose purpose-1 uniform draws the extra token
        u_add = (numpy_block([3, j, 0, 0], [seed, 0])[1] >> 11) / 2.0**53
        _, p, _ = ora.profile(target[0, j - 1], 1000, 0, 1000)
        if a < M:
            _, q, _ = ora.profile(draft[0, j - 1], 1000, 0, 1000)
            w = [max(Fraction(float(p[y])) - Fraction(float(q[y])), Fraction(0)) for y in range(V)]
        else:
            w = [Fraction(float(v)) for v in p]
        S = sum(w)
        t = Fraction(u_add) * S
        C, pick = Fraction(0), None
        for y in range(V):
            C += w[y]
            if C > t:
                pick = y
                break
        if out["d_cdf"][0] > 1e-12:
            assert out["out_tokens"][0, a] == pick
            checked += 1
    assert checked > 190
