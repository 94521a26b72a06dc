"""Pins for the oracle's commit step (ov_commit, ov_prefix_digest,
ov_contract_digest): SDCP Sec. 4.1-4.2 (digests), Sec. 6.3 steps 6-8
(truncation and commit) and Sec. 6.5 (low rounds, fallback ladder, m_cap).

References used: the values SDCP Appendix A prints (contract digest, d[0..2],
the worked greedy round), Python's hashlib for the digest chain, and action
sequences worked out by hand from the text of Sec. 6.5.2.
"""
import hashlib
import json
import os
import struct

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CONT, RED, SW, SELF, FIN, FAIL = range(6)


def appendix_a():
    return json.load(open(os.path.join(GOLDEN, "sdcp_appendix_a_digests.json")))


def chain(d, tokens):
    for t in tokens:
        d = hashlib.sha256(d + struct.pack(">I", t)).digest()
    return d


def run(contract, state, m, a, out, ok=None):
    return oracle.commit(contract, state, m, a, out, ok)


def test_appendix_a_contract_digest_and_prefix_chain():
    g = appendix_a()
    cd = oracle.contract_digest(bytes.fromhex(g["contract_cbor_hex"]))
    assert cd.hex() == g["contract_digest"]
    d0 = oracle.prefix_digest(cd, g["prompt"])
    assert d0.hex() == g["d"][0]
    # the two committed outputs, as two rounds of one token each
    k = oracle.make_contracts(1)
    s = oracle.make_states(1, digest=d0, n=0)
    for r, tok in enumerate(g["outputs"], start=1):
        out, e, act = run(k, s, [1], [0], [[tok, -1]])
        assert e[0] == 1 and s["n"][0] == r
        assert bytes(s["digest"][0]).hex() == g["d"][r]
    # and as one round committing both
    s = oracle.make_states(1, digest=d0, n=0)
    out, e, act = run(k, s, [1], [1], [g["outputs"]])
    assert e[0] == 2 and bytes(s["digest"][0]).hex() == g["d"][2]


def test_appendix_a_greedy_round():
    """n = 2; proposal [7, 9, 11]; target argmax 7, 9, 13, then 5: a = 2,
    emitted [7, 9, 13], new n = 5; not low, so c is reset and the action is
    continue."""
    g = appendix_a()
    rnd = json.load(open(os.path.join(GOLDEN, "sdcp_appendix_a_greedy_round.json")))
    d2 = bytes.fromhex(g["d"][2])
    k = oracle.make_contracts(1, m_max=8, max_new=256, low_rounds=3, stop=(2,),
                              fallback=(RED, SW, SELF, FAIL))
    s = oracle.make_states(1, digest=d2, n=rnd["committed_n"], m_cap=8)
    s["c"] = 2  # two low rounds before: this round resets c
    out, e, act = run(k, s, [3], [rnd["expected_accepted"]], [[7, 9, 13, -1]])
    assert out[0].tolist() == rnd["expected_emitted"] + [-1]
    assert e[0] == 3 and s["n"][0] == rnd["expected_new_committed"]
    assert act[0] == CONT and s["c"][0] == 0 and s["g"][0] == 1
    assert bytes(s["digest"][0]) == chain(d2, rnd["expected_emitted"])


def test_truncation_after_the_first_stop_token_and_at_max_new():
    k = oracle.make_contracts(6, max_new=256, stop=(2, 99))
    s = oracle.make_states(6, digest=b"\x11" * 32, n=10)
    s["n"][4] = 250
    s["n"][5] = 256
    out = np.array([[5, 2, 9, 4, -1],      # stop inside: committed through it
                    [5, 6, 7, 99, -1],     # the additional token is a stop token
                    [99, 2, 1, 1, -1],     # the first stop token wins
                    [5, 6, 7, 8, 3],       # no stop: all five committed
                    [1, 3, 4, 5, 6],       # max_new 256 from n = 250: six fit
                    [1, 3, -1, -1, -1]],   # n = max_new already: nothing fits
                   np.int32)
    a = np.array([3, 3, 3, 4, 4, 1], np.int32)
    res, e, act = run(k, s, [4] * 6, a, out)
    assert e.tolist() == [2, 4, 1, 5, 5, 0]
    assert act.tolist() == [FIN, FIN, FIN, CONT, CONT, FIN]
    assert res[0].tolist() == [5, 2, -1, -1, -1]
    assert res[2].tolist() == [99, -1, -1, -1, -1]
    assert s["n"].tolist() == [12, 14, 11, 15, 255, 256]
    assert bytes(s["digest"][1]) == chain(b"\x11" * 32, [5, 6, 7, 99])
    assert bytes(s["digest"][5]) == b"\x11" * 32
    # one more token: the session at 255 reaches max_new exactly
    res, e, act = run(k[4:5], s[4:5], [2], [2], [[8, 8, 8]])
    assert e[0] == 1 and act[0] == FIN and s["n"][4] == 256
    # six tokens that end exactly at max_new also finish generation
    s2 = oracle.make_states(1, n=250)
    res, e, act = run(k[:1], s2, [5], [5], [[3, 4, 5, 6, 7, 8]])
    assert e[0] == 6 and act[0] == FIN and s2["n"][0] == 256


def test_failed_session_commits_nothing():
    k = oracle.make_contracts(2)
    s = oracle.make_states(2, digest=b"\x22" * 32, n=7, m_cap=5)
    s["c"], s["g"], s["j"] = 1, 0, 2
    before = s.copy()
    res, e, act = run(k, s, [3, 3], [-1, 4], [[-1] * 4, [5] * 4])  # a = 4 > M = 3
    assert e.tolist() == [0, 0] and act.tolist() == [-1, -1]
    assert s.tobytes() == before.tobytes()


def rounds(k, s, seq, m=4, ok=None):
    """Run one session through rounds with accepted counts seq; returns the
    actions and the m_cap after each round."""
    acts, caps, js = [], [], []
    for a in seq:
        out = [[5] * (a + 1) + [-1] * (m - a)]
        _, _, act = run(k, s, [m], [a], out, None if ok is None else [ok])
        acts.append(int(act[0]))
        caps.append(int(s["m_cap"][0]))
        js.append(int(s["j"][0]))
    return acts, caps, js


def test_fallback_ladder_by_hand():
    """R = 3, ladder [reduce, switch, self_decode, fail], self_decode not
    permitted.  Every third consecutive low round applies the next entry:
    reduce (m_cap 8 -> 4), switch, then self_decode is skipped and fail is
    applied; with no entry left, fail again.  Three rounds that are not low
    reset j and restore m_cap by one each; the ladder then starts over."""
    k = oracle.make_contracts(1, m_max=8, low_rounds=3, stop=(),
                              fallback=(RED, SW, SELF, FAIL))
    s = oracle.make_states(1, m_cap=8)
    acts, caps, js = rounds(k, s, [0] * 12 + [3, 3, 3] + [0, 0, 0])
    assert acts == [CONT, CONT, RED, CONT, CONT, SW, CONT, CONT, FAIL, CONT, CONT, FAIL,
                    CONT, CONT, CONT, CONT, CONT, RED]
    assert caps == [8, 8, 4, 4, 4, 4, 4, 4, 4, 4, 4, 4, 5, 6, 7, 7, 7, 3]
    assert js == [0, 0, 1, 1, 1, 2, 2, 2, 4, 4, 4, 4, 4, 4, 0, 0, 0, 1]


def test_self_decode_applied_when_permitted_and_interrupted_runs():
    k = oracle.make_contracts(1, m_max=8, low_rounds=2, stop=(),
                              fallback=(SELF, RED, FAIL))
    s = oracle.make_states(1, m_cap=6)
    # low, not low (c reset), low, low -> self_decode (permitted)
    acts, caps, js = rounds(k, s, [0, 2, 0, 0], ok=1)
    assert acts == [CONT, CONT, CONT, SELF] and js[-1] == 1
    assert caps == [6, 7, 7, 7]
    # not permitted: skipped, reduce applied instead (j advances past both)
    s = oracle.make_states(1, m_cap=6)
    acts, caps, js = rounds(k, s, [0, 0], ok=0)
    assert acts == [CONT, RED] and js[-1] == 2 and caps[-1] == 3


def test_low_ratio():
    """low_ratio 50 with m = 4: low iff 100 a < 200, i.e. a <= 1."""
    k = oracle.make_contracts(1, low_rounds=1, low_ratio=50, stop=(), fallback=(RED,) * 8)
    s = oracle.make_states(1, m_cap=8)
    acts, caps, _ = rounds(k, s, [1, 2, 0, 4])
    assert acts == [RED, CONT, RED, CONT]
    assert caps == [4, 5, 2, 3]


def test_finish_takes_precedence_and_counters_still_move():
    k = oracle.make_contracts(1, low_rounds=1, stop=(2,), fallback=(RED,))
    s = oracle.make_states(1, m_cap=8)
    _, e, act = run(k, s, [4], [0], [[2, -1, -1, -1, -1]])  # a = 0 (low), token 2 stops
    assert act[0] == FIN and e[0] == 1 and s["m_cap"][0] == 4 and s["j"][0] == 1
