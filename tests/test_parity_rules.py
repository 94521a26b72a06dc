"""The parity bar's own rules, on hand-made results (no GPU): a session that
differs from the oracle is excused only by the delta of the first decision at
which it departs (the acceptance test at that position, a top-p cut of a row
that decision reads, or the additional token's inverse CDF), never by a
near-tie elsewhere in the session; near-ties are counted by kind over the
decisions the oracle took."""
import numpy as np
import pytest

import oracle
from tests import parity

INF = np.inf


def results(B=2, M=4, a=(2, 1)):
    """An oracle result and a GPU copy of it, with every delta far from 0."""
    o = {
        "accepted_len": np.array(a, np.int32),
        "out_tokens": np.full((B, M + 1), -1, np.int32),
        "p_tok": np.full((B, M), 0.2), "q_tok": np.full((B, M), 0.3),
        "d_acc": np.full((B, M), 0.1), "d_topp_t": np.full((B, M + 1), 0.1),
        "d_topp_d": np.full((B, M), 0.1), "d_cdf": np.full(B, 0.1),
    }
    for b in range(B):
        o["out_tokens"][b, :a[b] + 1] = np.arange(a[b] + 1) + 10
    g = {k: o[k].copy() for k in ("accepted_len", "out_tokens", "p_tok", "q_tok")}
    return g, o


def test_identical_results_pass():
    g, o = results()
    rep = parity.compare(g, o, "same")
    assert rep["mismatches"] == 0 and sum(rep["excused"].values()) == 0


def test_acceptance_near_tie_at_the_deciding_position_is_excused():
    g, o = results()
    g["accepted_len"][0] = 3            # the GPU accepted position 3, the oracle rejected it
    g["out_tokens"][0, 2:4] = [12, 99]
    o["d_acc"][0, 2] = 4e-7
    rep = parity.compare(g, o, "acc")
    assert rep["excused"] == {"acc": 1, "topp": 0, "cdf": 0}


def test_a_near_tie_elsewhere_does_not_excuse():
    g, o = results()
    g["accepted_len"][0] = 3
    g["out_tokens"][0, 2:4] = [12, 99]
    o["d_acc"][0, 2] = 1e-3             # the deciding test is far from its threshold
    o["d_topp_t"][0, 3] = 1e-9          # a near-tie in a later row
    o["d_acc"][0, 0] = 1e-9             # and at an earlier, agreeing position
    o["d_cdf"][0] = 1e-9
    with pytest.raises(AssertionError, match="unexcused"):
        parity.compare(g, o, "elsewhere")


def test_support_membership_difference_is_a_top_p_decision():
    g, o = results()
    g["accepted_len"][1] = 0            # x_2 outside p_2's support on the GPU
    g["out_tokens"][1, :2] = [77, -1]
    g["p_tok"][1, 0] = 0.0
    o["d_acc"][1, 0] = 1e-9             # not this test: the cut decided it
    o["d_topp_t"][1, 0] = 1e-3
    with pytest.raises(AssertionError, match="unexcused"):
        parity.compare(g, o, "member-far")
    o["d_topp_t"][1, 0] = 2e-7
    rep = parity.compare(g, o, "member-near")
    assert rep["excused"]["topp"] == 1


def test_additional_token_excused_by_its_cdf_only():
    g, o = results()
    g["out_tokens"][0, 2] = 55          # same a, another additional token
    o["d_cdf"][0] = 5e-2
    o["d_acc"][0, 3] = 1e-9             # a position after the deciding one
    with pytest.raises(AssertionError, match="unexcused"):
        parity.compare(g, o, "cdf-far")
    o["d_cdf"][0] = 3e-7
    rep = parity.compare(g, o, "cdf-near")
    assert rep["excused"]["cdf"] == 1


def test_statuses():
    g, o = results()
    g["accepted_len"][0] = oracle.S_BAD_PROPOSAL
    g["out_tokens"][0] = -1
    g["p_tok"][0] = g["q_tok"][0] = -1.0
    o["d_topp_d"][0, 1] = 5e-7          # a drafted token at its draft row's cut
    parity.compare(g, o, "bad-proposal-near")
    o["d_topp_d"][0, 1] = 1e-2
    with pytest.raises(AssertionError):
        parity.compare(g, o, "bad-proposal-far")
    g2, o2 = results()
    g2["accepted_len"][1] = oracle.S_BAD_LOGITS
    g2["out_tokens"][1] = -1
    o2["d_topp_d"][1] = 0.0             # no near-tie excuses a bad-logits difference
    with pytest.raises(AssertionError):
        parity.compare(g2, o2, "bad-logits")


def test_near_ties_counted_over_decisions_taken():
    _, o = results(a=(2, 1))
    o["d_acc"][0, 2] = 1e-8             # session 0 decides at position 3: counted
    o["d_acc"][0, 3] = 1e-8             # after the decision: not counted
    o["d_topp_t"][1, 1] = 1e-8          # session 1's deciding row: counted
    o["d_topp_t"][1, 4] = 1e-8          # a row it never decided on: not counted
    o["d_cdf"][1] = 1e-8
    assert parity.near_ties(o) == {"acc": 1, "topp": 1, "cdf": 1}


def test_probability_tolerance():
    g, o = results()
    g["p_tok"][0, 0] *= 1 + 3e-7
    parity.compare(g, o, "rtol-default")
    with pytest.raises(AssertionError, match="probability"):
        parity.compare(g, o, "rtol-tight", prob_rtol=2e-7)


def test_probability_at_a_near_tie_cut_is_excused_and_counted():
    g, o = results()
    g["p_tok"][0, 1] *= 1 + 3e-6        # the row's support holds one token more
    with pytest.raises(AssertionError, match="probability"):
        parity.compare(g, o, "cut-far", prob_rtol=2e-7)
    o["d_topp_t"][0, 1] = 4e-9          # the oracle's cut of that row is a near-tie
    rep = parity.compare(g, o, "cut-near", prob_rtol=2e-7)
    assert rep["prob_at_near_tie_cut"] == 1
    o["d_topp_t"][0, 1] = 0.1
    o["d_topp_d"][0, 1] = 4e-9          # a near-tie of the draft row excuses q only
    with pytest.raises(AssertionError, match="probability"):
        parity.compare(g, o, "cut-other-row", prob_rtol=2e-7)
