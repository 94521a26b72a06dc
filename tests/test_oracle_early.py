"""Pins for the oracle's in-order reading (ov_verify_early): positions are
examined one after another and each row is read only when its position is
reached (textbook "The acceptance rule": the first rejection ends the round),
where the SDCP reading (Sec. 6.3 step 5) checks every row and every
q_i(x_i) before any decision.

References used: the SDCP reading of the oracle (ov_verify, ov_verify_sdcp,
ov_verify_qrows), pinned by its own tests.  On a session whose rows are all
usable and whose q_i(x_i) are all positive both readings must give the same
verdict, since a rejection decided at position j depends on rows 1..j only;
rows after the deciding position, overwritten with NaN, must change nothing
in the in-order reading while the SDCP reading fails on them; a problem at or
before the deciding position fails the session in both.
"""
import numpy as np
import pytest

from tests import parity

RELAXED = 192


def mixed_case(ora, seed, B=36, M=6, V=300, q_source="draft", sdcp=False):
    """Sessions of every rule and profile, with drafts close enough to the
    target that acceptance lengths spread over 0..M."""
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 1.5, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.6, size=(B, M, V))).astype(np.float32)
    s = ora.make_sampling(B, 1000, 0, 1000)
    profiles = [(1000, 0, 1000), (700, 20, 1000), (900, 0, 850), (1200, 50, 900), (0, 0, 1000)]
    rules = [2, 2, 1, RELAXED, 2, 2]
    for b in range(B):
        s[b]["temperature_milli"], s[b]["top_k"], s[b]["top_p_milli"] = profiles[b % 5]
    h = dict(target=t, draft=d, tokens=np.zeros((B, M), np.int32),
             m=rng.integers(1, M + 1, size=B).astype(np.int32),
             rule=np.array([rules[b % 6] for b in range(B)], np.int32), sampling=s,
             seed=int(rng.integers(0, 1 << 62)), round=int(rng.integers(1, 50)))
    h["tokens"] = parity.draw_valid_tokens(h, rng)
    if q_source == "qrows":
        q = np.exp(d.astype(np.float64) - d.max(axis=-1, keepdims=True))
        q /= q.sum(axis=-1, keepdims=True)
        h["q_rows"] = q.astype(np.float32)
        h["draft"] = None
    if sdcp:
        h["sdcp"] = parity.random_sdcp_sessions(B, rng)
    return h


def run(ora, h, early):
    return ora.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"],
                      h["seed"], h["round"], sdcp_sessions=h.get("sdcp"), q_rows=h.get("q_rows"),
                      early=early)


def assert_same_verdict(e, f, b, M):
    a = int(f["accepted_len"][b])
    assert e["accepted_len"][b] == a, b
    assert np.array_equal(e["out_tokens"][b], f["out_tokens"][b]), b
    # probes up to the deciding position (a + 1), -1 after
    upto = min(a + 1, M)
    for name in ("p_tok", "q_tok"):
        assert np.array_equal(e[name][b, :upto], f[name][b, :upto]), (name, b)
        assert (e[name][b, upto:] == -1).all(), (name, b)


CASES = [("draft", False), ("qrows", False), ("draft", True), ("qrows", True)]


@pytest.mark.parametrize("q_source,sdcp", CASES)
def test_same_verdict_where_every_row_is_usable(ora, q_source, sdcp):
    h = mixed_case(ora, 11 + len(q_source) + sdcp, q_source=q_source, sdcp=sdcp)
    f, e = run(ora, h, False), run(ora, h, True)
    a = f["accepted_len"]
    assert (a >= 0).sum() >= 24 and len(set(a[a >= 0].tolist())) >= 4, "spread of lengths"
    M = h["tokens"].shape[1]
    for b in range(len(a)):
        if a[b] >= 0:
            assert_same_verdict(e, f, b, M)
        else:  # a failing session fails in order too, at the same or a later problem
            assert e["accepted_len"][b] < 0 or f["accepted_len"][b] == ora.S_BAD_PROPOSAL


@pytest.mark.parametrize("q_source,sdcp", CASES[:2])
def test_rows_after_the_deciding_position_are_not_read(ora, q_source, sdcp):
    """Every target row after a + 1 and every draft row (or published row)
    after a + 1 is overwritten with NaN: the in-order verdict is the clean
    SDCP verdict, and the SDCP reading now fails each session that had such
    a row."""
    h = mixed_case(ora, 21 + len(q_source), q_source=q_source, sdcp=sdcp)
    f = run(ora, h, False)
    a = f["accepted_len"]
    M = h["tokens"].shape[1]
    c = dict(h)
    c["target"] = h["target"].copy()
    key = "q_rows" if q_source == "qrows" else "draft"
    c[key] = h[key].copy()
    touched = []
    for b in range(len(a)):
        if a[b] < 0:
            continue
        e = int(a[b]) + 1  # deciding position, 1-based
        if e <= int(h["m"][b]):
            c["target"][b, e:] = np.nan
            c[key][b, e:] = np.nan
            touched.append(b)
    assert len(touched) >= 12
    e_run = run(ora, c, True)
    for b in range(len(a)):
        if a[b] >= 0:
            assert_same_verdict(e_run, f, b, M)
    f_bad = run(ora, c, False)
    for b in touched:
        assert f_bad["accepted_len"][b] < 0, b


def test_problems_at_or_before_the_deciding_position_fail(ora):
    """A NaN in target row j <= a + 1 fails the session with BAD_LOGITS; a zero
    q_j(x_j) (the drafted token's draft logit set to -inf) at j <= a + 1 with
    BAD_PROPOSAL, in both readings."""
    h = mixed_case(ora, 31)
    f = run(ora, h, False)
    a = f["accepted_len"]
    rng = np.random.default_rng(5)
    for b in np.nonzero(a >= 0)[0][:16]:
        e = int(a[b]) + 1
        j = int(rng.integers(1, e + 1))  # 1-based position at or before the deciding one
        c = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
        c["target"][b, j - 1, int(rng.integers(0, c["target"].shape[2]))] = np.nan
        assert run(ora, c, True)["accepted_len"][b] == ora.S_BAD_LOGITS
        assert run(ora, c, False)["accepted_len"][b] == ora.S_BAD_LOGITS
        if h["rule"][b] == 2 and j <= int(h["m"][b]):
            c = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
            c["draft"][b, j - 1, int(h["tokens"][b, j - 1])] = -np.inf
            assert run(ora, c, True)["accepted_len"][b] == ora.S_BAD_PROPOSAL
            assert run(ora, c, False)["accepted_len"][b] == ora.S_BAD_PROPOSAL


def test_greedy_in_order_is_the_argmax_prefix(ora):
    """Rule 1 read in order: the brute-force longest prefix matching the
    target argmax, then the argmax of the next row; rows after it NaN."""
    rng = np.random.default_rng(8)
    B, M, V = 40, 5, 64
    t = rng.integers(0, 6, size=(B, M + 1, V)).astype(np.float32)  # ties: smallest id wins
    am = np.argmax(t, axis=-1)
    tokens = np.where(rng.random((B, M)) < 0.75, am[:, :M], rng.integers(0, V, (B, M)))
    tokens = tokens.astype(np.int32)
    want_a = np.array([next((i for i in range(M) if tokens[b, i] != am[b, i]), M)
                       for b in range(B)])
    for b in range(B):
        t[b, want_a[b] + 1:] = np.nan
    e = ora.verify(t, None, tokens, [M] * B, [1] * B, ora.make_sampling(B, 1000, 0, 1000), 1, 1,
                   early=True)
    assert np.array_equal(e["accepted_len"], want_a)
    for b in range(B):
        a = want_a[b]
        assert np.array_equal(e["out_tokens"][b, :a], tokens[b, :a])
        assert e["out_tokens"][b, a] == am[b, a]
        assert (e["out_tokens"][b, a + 1:] == -1).all()


def test_bad_row_before_unusable_q_at_one_position(ora):
    """At one position a bad row and an unusable q_i(x_i) together fail the
    session with BAD_LOGITS (the row is read first); an unusable q_i(x_i)
    alone at an earlier position than a bad row gives BAD_PROPOSAL."""
    h = mixed_case(ora, 41)
    f = run(ora, h, False)
    a = f["accepted_len"]
    checked = 0
    for b in np.nonzero((a >= 1) & (h["rule"] == 2))[0][:8]:
        e = int(a[b]) + 1
        x1 = int(h["tokens"][b, 0])
        c = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
        c["target"][b, 0, 7] = np.nan                 # bad target row 1
        c["draft"][b, 0, x1] = -np.inf                # and q_1(x_1) = 0
        assert run(ora, c, True)["accepted_len"][b] == ora.S_BAD_LOGITS
        c = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
        c["draft"][b, 0, x1] = -np.inf                # q_1(x_1) = 0 ...
        c["target"][b, e - 1, 7] = np.nan             # ... before a bad row at e >= 2
        assert run(ora, c, True)["accepted_len"][b] == ora.S_BAD_PROPOSAL
        # the SDCP reading checks every row first
        assert run(ora, c, False)["accepted_len"][b] == ora.S_BAD_LOGITS
        checked += 1
    assert checked >= 3
