"""Pins for the oracle's relaxed rule (rule 192, a private-use value of the
SDCP rule registry, Sec. 10.2.2): relaxed acceptance by membership of the
target's top-k (textbook "Inference: KV Cache, Batching, Speculative
Decoding", section "Speculative decoding"), read as: accept x_i while
p_i(x_i) > 0, then draw the additional token from p_{a+1} with the purpose-1
value of position a+1.

References used: brute-force top-k membership with numpy's ordering (logit
descending, id ascending); Rule 1 (greedy) at temperature 0; numpy's Philox
and exact rationals for the draw; chi-square of the additional token against
p_{a+1}.
"""
from fractions import Fraction

import numpy as np

from tests.test_oracle_philox import numpy_block
from tests.test_oracle_stats import chisq_pvalue

RELAXED = 192


def topk_members(row, k):
    order = np.lexsort((np.arange(row.shape[0]), -row.astype(np.float64)))
    return set(order[:k].tolist())


def test_accepts_while_the_token_is_in_the_target_top_k(ora):
    rng = np.random.default_rng(40)
    B, M, V, k = 60, 6, 30, 5
    target = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, M)).astype(np.int32)
    # make membership likely at early positions
    for b in range(B):
        for i in range(M):
            if rng.random() < 0.7:
                tokens[b, i] = rng.choice(sorted(topk_members(target[b, i], k)))
    out = ora.verify(target, None, tokens, [M] * B, [RELAXED] * B,
                     ora.make_sampling(B, 800, k, 1000), 3, 2)
    for b in range(B):
        want = M
        for i in range(M):
            if tokens[b, i] not in topk_members(target[b, i], k):
                want = i
                break
        assert out["accepted_len"][b] == want, b
        assert np.array_equal(out["out_tokens"][b, :want], tokens[b, :want])
        assert out["out_tokens"][b, want] in topk_members(target[b, want], k)
        assert (out["q_tok"][b] == -1).all()


def test_temperature_zero_equals_greedy(ora):
    rng = np.random.default_rng(41)
    B, M, V = 40, 5, 50
    target = rng.normal(0, 1, size=(B, M + 1, V)).astype(np.float32)
    tokens = np.argmax(target[:, :M], axis=-1).astype(np.int32)
    flip = rng.random((B, M)) < 0.3
    tokens[flip] = rng.integers(0, V, size=flip.sum())
    s = ora.make_sampling(B, 0, 0, 1000)
    r = ora.verify(target, None, tokens, [M] * B, [RELAXED] * B, s, 9, 1)
    g = ora.verify(target, None, tokens, [M] * B, [1] * B, s, 9, 1)
    assert np.array_equal(r["accepted_len"], g["accepted_len"])
    assert np.array_equal(r["out_tokens"], g["out_tokens"])


def test_additional_token_is_the_exact_inverse_cdf_of_p_next(ora):
    rng = np.random.default_rng(42)
    V, M, k = 9, 3, 4
    checked = 0
    for trial in range(200):
        target = rng.normal(0, 1, size=(1, M + 1, V)).astype(np.float32)
        tokens = rng.integers(0, V, size=(1, M)).astype(np.int32)
        seed = int(rng.integers(0, 1 << 62))
        out = ora.verify(target, None, tokens, [M], [RELAXED], ora.make_sampling(1, 1000, k, 1000),
                         seed, 5)
        a = int(out["accepted_len"][0])
        u = (numpy_block([5, a + 1, 0, 0], [seed, 0])[1] >> 11) / 2.0**53
        _, p, _ = ora.profile(target[0, a], 1000, k, 1000)
        w = [Fraction(float(v)) for v in p]
        t = Fraction(u) * sum(w)
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


def test_additional_token_follows_p_of_its_position(ora):
    """Given the first non-member position j, the additional token follows p_j
    (the rule does not preserve the target distribution for the accepted
    tokens, but the token it samples is the target's own)."""
    rng = np.random.default_rng(43)
    V, M, n, k = 8, 2, 40_000, 3
    rows = rng.normal(0, 1, size=(M + 1, V)).astype(np.float32)
    out_of_topk = sorted(set(range(V)) - topk_members(rows[0], k))
    tokens = np.zeros((n, M), np.int32)
    tokens[:, 0] = rng.choice(out_of_topk, size=n)  # always rejected at position 1
    tokens[:, 1] = 0
    out = ora.verify(np.broadcast_to(rows, (n, M + 1, V)).copy(), None, tokens, [M] * n,
                     [RELAXED] * n, ora.make_sampling(n, 1000, k, 1000), 77, 1, diagnostics=False)
    assert (out["accepted_len"] == 0).all()
    p = ora.profile(rows[0], 1000, k, 1000)[1]
    counts = np.bincount(out["out_tokens"][:, 0], minlength=V)
    assert chisq_pvalue(counts, p) > 1e-3


def test_members_with_tiny_probability_are_accepted(ora):
    """At T = 0.05 the k-th member of the top-k has p ~ exp(-20 * gap): tiny but
    positive, so it is accepted; the next token is not a member."""
    V, M, k = 12, 2, 4
    row = np.array([3.0, 2.0, 1.5, 1.0, 0.5, 0.0, -1, -2, -3, -4, -5, -6], np.float32)
    target = np.broadcast_to(row, (1, M + 1, V)).copy()
    s = ora.make_sampling(1, 50, k, 1000)
    out = ora.verify(target, None, np.array([[3, 4]], np.int32), [M], [RELAXED], s, 1, 1)
    assert 0 < out["p_tok"][0, 0] < 1e-12
    assert out["accepted_len"][0] == 1 and out["p_tok"][0, 1] == 0.0
