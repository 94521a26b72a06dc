"""Pins for the oracle's sampling profile (SDCP Sec. 4.1: temperature, then
top-k, then top-p; temperature 0 is the argmax with ties to the smallest id)
and for its inverse-CDF sampler.

Each check compares the oracle with something other than itself: a library
routine (torch / scipy softmax, numpy's stable argsort, numpy argmax), exact
rational arithmetic (fractions), or a brute-force enumeration on tiny rows.
The tie readings (exactly k tokens for top-k in the order (logit desc, id
asc); an inclusive top-p boundary 1000*C >= P*Z_k) are not fixed by the
pages; these tests pin the oracle's implementation of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import softmax


def f32(a):
    return np.asarray(a, dtype=np.float32)


def test_untruncated_profile_is_softmax_at_temperature(ora):
    rng = np.random.default_rng(1)
    for t_milli in (1, 250, 700, 1000, 2500, 40000):
        row = f32(rng.normal(0, 3, size=777))
        st, p, d = ora.profile(row, t_milli, 0, 1000)
        assert st == 0 and d == math.inf
        ref = torch.softmax(torch.from_numpy(row.astype(np.float64)) / (t_milli / 1000.0), 0).numpy()
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)


def test_top_k_at_or_above_finite_count_is_off(ora):
    rng = np.random.default_rng(2)
    row = f32(rng.normal(0, 1, size=64))
    _, p_off, _ = ora.profile(row, 1000, 0, 1000)
    for k in (64, 65, 10**9):
        _, p, _ = ora.profile(row, 1000, k, 1000)
        assert np.array_equal(p, p_off)


def test_temperature_zero_is_one_hot_argmax_smallest_id(ora):
    row = f32([0.5, 3.0, -1.0, 3.0, 3.0, 2.9])
    st, p, _ = ora.profile(row, 0, 0, 1000)
    assert st == 0
    assert p.tolist() == [0, 1, 0, 0, 0, 0]
    rng = np.random.default_rng(3)
    for _ in range(50):
        row = f32(rng.integers(-3, 3, size=40))  # many ties
        _, p, _ = ora.profile(row, 0, 17, 300)
        assert p[np.argmax(row)] == 1.0 and p.sum() == 1.0


def test_minus_inf_has_zero_probability(ora):
    rng = np.random.default_rng(4)
    row = f32(rng.normal(0, 2, size=100))
    row[rng.choice(100, 30, replace=False)] = -np.inf
    st, p, _ = ora.profile(row, 800, 0, 1000)
    assert st == 0
    ref = torch.softmax(torch.from_numpy(row.astype(np.float64)) / 0.8, 0).numpy()
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=0)
    assert np.all(p[np.isinf(row)] == 0)


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_nan_or_plus_inf_is_bad_logits(ora, bad):
    row = f32([0.0, 1.0, bad, 2.0])
    st, _, _ = ora.profile(row, 1000, 0, 1000)
    assert st == ora.S_BAD_LOGITS


def test_all_minus_inf_is_bad_logits(ora):
    st, _, _ = ora.profile(f32([-np.inf] * 5), 1000, 0, 1000)
    assert st == ora.S_BAD_LOGITS
    st, _, _ = ora.profile(f32([-np.inf] * 5), 0, 0, 1000)
    assert st == ora.S_BAD_LOGITS


def test_signed_zeros_are_equal_logits(ora):
    row = f32([-0.0, 0.0, -1.0])
    _, p, _ = ora.profile(row, 0, 0, 1000)
    assert p.tolist() == [1.0, 0.0, 0.0]  # tie -> smallest id
    _, p, _ = ora.profile(row, 1000, 1, 1000)
    assert p.tolist() == [1.0, 0.0, 0.0]
    _, p, _ = ora.profile(row, 1000, 0, 1000)
    assert p[0] == p[1]


def library_top_k(row, t_milli, k):
    order = np.argsort(-row.astype(np.float64), kind="stable")  # ties: ascending id
    finite = order[np.isfinite(row[order])]
    keep = finite[:k] if 0 < k < len(finite) else finite
    p = np.zeros(row.shape[0])
    p[keep] = softmax(row[keep].astype(np.float64) / (t_milli / 1000.0))
    return p


def test_top_k_matches_stable_argsort_and_softmax(ora):
    rng = np.random.default_rng(5)
    for trial in range(200):
        V = int(rng.integers(1, 300))
        row = f32(np.round(rng.normal(0, 2, size=V) * 4) / 4)  # plenty of ties
        if trial % 3 == 0:
            row[rng.random(V) < 0.2] = -np.inf
            if np.all(np.isinf(row)):
                row[0] = 0.0
        k = int(rng.integers(1, V + 3))
        t = int(rng.integers(1, 3000))
        st, p, _ = ora.profile(row, t, k, 1000)
        assert st == 0
        np.testing.assert_allclose(p, library_top_k(row, t, k), rtol=1e-12, atol=0)
        n_finite = int(np.isfinite(row).sum())
        assert int((p > 0).sum()) <= min(k, n_finite)


def brute_force_profile(row, t_milli, k, p_milli):
    """Enumerate prefix lengths of the order with exact sums (math.fsum)."""
    V = row.shape[0]
    ids = sorted((i for i in range(V) if np.isfinite(row[i])),
                 key=lambda i: (-float(row[i]), i))
    if 0 < k < len(ids):
        ids = ids[:k]
    lmax = float(row[ids[0]])
    w = [math.exp((float(row[i]) - lmax) / (t_milli / 1000.0)) for i in ids]
    Zk = math.fsum(w)
    L = len(ids)
    if p_milli < 1000:
        L = next(n for n in range(1, len(ids) + 1)
                 if 1000.0 * math.fsum(w[:n]) >= p_milli * Zk)
    p = np.zeros(V)
    Z = math.fsum(w[:L])
    for j in range(L):
        p[ids[j]] = w[j] / Z
    return p, L


def test_top_p_matches_brute_force_prefix_search(ora):
    rng = np.random.default_rng(6)
    checked = 0
    for trial in range(400):
        V = int(rng.integers(1, 60))
        row = f32(rng.normal(0, 1.5, size=V))
        k = int(rng.integers(0, V + 2))
        t = int(rng.integers(100, 2000))
        P = int(rng.integers(0, 1000))
        st, p, d = ora.profile(row, t, k, P)
        assert st == 0
        if d < 1e-9:
            continue  # the boundary is too close to decide from rounded sums
        ref, L = brute_force_profile(row, t, k, P)
        assert int((p > 0).sum()) == L
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=0)
        checked += 1
    assert checked > 350


def test_top_p_boundary_is_inclusive_and_ties_break_by_id(ora):
    # four equal weights: mass after two tokens is exactly half
    row = f32([1.0, 1.0, 1.0, 1.0])
    _, p, d = ora.profile(row, 1000, 0, 500)
    assert p.tolist() == [0.5, 0.5, 0.0, 0.0]  # 1000*2 >= 500*4 keeps exactly two
    assert d == 0.0
    _, p, _ = ora.profile(row, 1000, 0, 501)
    assert p.tolist() == pytest.approx([1 / 3, 1 / 3, 1 / 3, 0.0], rel=1e-15)
    # top_p = 0 keeps only the first token of the order
    row = f32([0.2, 0.9, 0.9, -3.0])
    _, p, _ = ora.profile(row, 1000, 0, 0)
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0]
    # top_k = 1 as well
    _, p, _ = ora.profile(row, 1000, 1, 1000)
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0]


def test_top_p_is_measured_after_top_k(ora):
    # weights at T=ln-scaled logits: 0.4, 0.3, 0.2, 0.1 (exact ratios 4:3:2:1)
    row = f32(np.log([4.0, 3.0, 2.0, 1.0]))
    # top-k=2 renormalises to 4/7, 3/7; top-p 0.5 then keeps one token.
    # Applied to the full distribution, top-p 0.5 would keep two (0.4 < 0.5).
    _, p, _ = ora.profile(row, 1000, 2, 500)
    assert p.tolist() == [1.0, 0.0, 0.0, 0.0]
    _, p, _ = ora.profile(row, 1000, 0, 500)
    assert (p > 0).sum() == 2


def test_bf16_rows_widen_exactly(ora):
    rng = np.random.default_rng(8)
    x = rng.normal(0, 3, size=500).astype(np.float32)
    bits = ora.bf16_bits(x)
    wide = ora.bf16_to_float(bits)
    # numpy-free reference for the widening: torch's bfloat16 -> float32
    tb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(wide, tb)
    for args in [(700, 50, 900), (1000, 0, 950), (0, 0, 1000), (1300, 7, 1000)]:
        s1, p1, _ = ora.profile(bits, *args)
        s2, p2, _ = ora.profile(wide, *args)
        assert s1 == s2 == 0
        assert np.array_equal(p1, p2)


def exact_inverse_cdf(w, u):
    wf = [Fraction(float(v)) for v in w]
    S = sum(wf)
    t = Fraction(float(u)) * S
    C = Fraction(0)
    for y, v in enumerate(wf):
        C += v
        if C > t:
            return y
    return max(y for y, v in enumerate(wf) if v > 0)


def test_inverse_cdf_matches_exact_rationals(ora):
    rng = np.random.default_rng(9)
    for _ in range(500):
        V = int(rng.integers(1, 20))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[rng.integers(0, V)] = 0.3
        u = float(rng.random())
        y, d = ora.inverse_cdf(w, u)
        if d > 1e-12:
            assert y == exact_inverse_cdf(w, u)
        assert w[y] > 0


def test_inverse_cdf_boundaries(ora):
    w = np.array([0.25, 0.0, 0.25, 0.5])
    assert ora.inverse_cdf(w, 0.0)[0] == 0
    assert ora.inverse_cdf(w, 0.25)[0] == 2  # C_0 = 0.25 is not > 0.25; id 1 has no mass
    assert ora.inverse_cdf(w, 0.5)[0] == 3
    assert ora.inverse_cdf(w, 1.0 - 2**-53)[0] == 3


def test_residual_pick_is_inverse_cdf_of_positive_part(ora):
    rng = np.random.default_rng(10)
    for _ in range(300):
        V = int(rng.integers(2, 12))
        p = rng.dirichlet(np.ones(V))
        q = rng.dirichlet(np.ones(V))
        u = float(rng.random())
        y, d = ora.residual_pick(p, q, u)
        w = np.maximum(p - q, 0)
        if d > 1e-12:
            assert y == exact_inverse_cdf(w, u)
        assert p[y] > q[y]


def test_residual_without_mass_falls_back_to_p(ora):
    p = np.array([0.25, 0.0, 0.75])
    q = p.copy()  # max(0, p - q) has no mass (reachable only through rounding)
    assert ora.residual_pick(p, q, 0.1)[0] == 0
    assert ora.residual_pick(p, q, 0.3)[0] == 2
    q = np.array([0.25, 0.1, 0.75])  # p <= q everywhere
    assert ora.residual_pick(p, q, 0.9)[0] == 2
