"""Pins of the oracle's SDCP uniforms (SDCP Sec. 6.4): its own SHA-256
(FIPS 180-4) against the digests SDCP Appendix A prints and against Python's
hashlib, its HMAC (RFC 2104) against Python's hmac, and the derivation of the
two verifier values from the MAC."""
import hashlib
import hmac
import json
import os
import struct

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sdcp_appendix_a_digests.json")


def u32(x):
    return struct.pack(">I", x)


def test_sha256_appendix_a_contract_digest():
    g = json.load(open(GOLDEN))
    cbor = bytes.fromhex(g["contract_cbor_hex"])
    assert len(cbor) == g["contract_cbor_len"] == 143
    # Sec. 4.1: SHA-256("SDCP-CONTRACT-1" || 0x00 || deterministic CBOR)
    cd = oracle.sha256(b"SDCP-CONTRACT-1\x00" + cbor)
    assert cd.hex() == g["contract_digest"]


def test_sha256_appendix_a_prefix_chain():
    g = json.load(open(GOLDEN))
    cd = bytes.fromhex(g["contract_digest"])
    prompt = g["prompt"]
    # Sec. 4.2: d[0] over the domain separator, contract digest, P and the prompt
    d = oracle.sha256(b"SDCP-PREFIX-1\x00" + cd + u32(len(prompt)) + b"".join(u32(t) for t in prompt))
    assert d.hex() == g["d"][0]
    for k, o in enumerate(g["outputs"], start=1):
        d = oracle.sha256(d + u32(o))
        assert d.hex() == g["d"][k]


@pytest.mark.parametrize("n", [0, 1, 3, 54, 55, 56, 57, 63, 64, 65, 119, 120, 127, 128, 129, 200, 1000])
def test_sha256_matches_hashlib_at_padding_boundaries(n):
    msg = bytes((7 * i + n) & 0xFF for i in range(n))
    assert oracle.sha256(msg) == hashlib.sha256(msg).digest()


def test_hmac_matches_python_hmac():
    rng = np.random.default_rng(3)
    for klen in (0, 1, 8, 32, 63, 64, 65, 100):
        for mlen in (0, 1, 39, 64, 200):
            key = rng.integers(0, 256, klen, dtype=np.uint8).tobytes()
            msg = rng.integers(0, 256, mlen, dtype=np.uint8).tobytes()
            assert oracle.hmac_sha256(key, msg) == hmac.new(key, msg, hashlib.sha256).digest()


def test_sdcp_uniform_message_layout_and_53_bits():
    """Sec. 6.4: key = seed as 8 octets network order; message "SDCP-VERIFY-1"
    || 0x00 || session || uint32(round) || uint32(i) || uint8(purpose); value =
    first 53 bits of the MAC / 2^53."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        session = rng.integers(0, 256, 16, dtype=np.uint8).tobytes()
        rnd = int(rng.integers(0, 2**32))
        i = int(rng.integers(1, 66))
        for purpose in (0, 1):
            msg = b"SDCP-VERIFY-1\x00" + session + u32(rnd) + u32(i) + bytes([purpose])
            mac = hmac.new(struct.pack(">Q", seed), msg, hashlib.sha256).digest()
            want = (int.from_bytes(mac[:8], "big") >> 11) / 2.0**53
            got = oracle.sdcp_uniform(seed, session, rnd, i, purpose)
            assert got == want
            assert 0.0 <= got < 1.0 and (got * 2**53).is_integer()


def test_sdcp_uniforms_are_uniform():
    session = bytes(range(16))
    u = [oracle.sdcp_uniform(12345, session, r, i, p) for r in range(1, 101) for i in range(1, 51)
         for p in (0, 1)]
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    assert len(set(u)) == len(u)


def _small_batch(rng, B=24, M=4, V=12):
    t = rng.normal(0, 1.5, size=(B, M + 1, V)).astype(np.float32)
    d = (t[:, :M] + rng.normal(0, 0.8, size=(B, M, V))).astype(np.float32)
    rule = np.where(np.arange(B) % 3 == 0, 1, 2).astype(np.int32)
    s = oracle.make_sampling(B, 900, 0, 950)
    h = dict(target=t, draft=d, m=np.full(B, M, np.int32), rule=rule, sampling=s)
    toks = np.zeros((B, M), np.int32)
    for b in range(B):
        for i in range(M):
            _, q, _ = oracle.profile(d[b, i], 900, 0, 950)
            toks[b, i] = rng.choice(V, p=q / q.sum())
    h["tokens"] = toks
    return h


def test_verify_sdcp_greedy_sessions_use_no_uniforms():
    rng = np.random.default_rng(11)
    h = _small_batch(rng)
    a = oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"], 7, 3)
    sess = oracle.make_sdcp_sessions(24, seed=99, round_=8)
    b = oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"], 0, 0,
                      sdcp_sessions=sess)
    greedy = h["rule"] == 1
    assert np.array_equal(a["accepted_len"][greedy], b["accepted_len"][greedy])
    assert np.array_equal(a["out_tokens"][greedy], b["out_tokens"][greedy])
    # p and q do not depend on the generator
    assert np.array_equal(a["p_tok"], b["p_tok"]) and np.array_equal(a["q_tok"], b["q_tok"])


def test_verify_sdcp_uses_the_session_values():
    """Rule 2 decisions follow the SDCP values of each session's (seed, id,
    round): u_acc(i) < min(1, p/q) accepts, recomputed here from the oracle's
    probabilities and uniforms."""
    rng = np.random.default_rng(12)
    h = _small_batch(rng)
    B, M = h["tokens"].shape
    sess = oracle.make_sdcp_sessions(B, seed=2024, round_=5)
    o = oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"], 0, 0,
                      sdcp_sessions=sess)
    for b in range(B):
        if h["rule"][b] != 2 or o["accepted_len"][b] < 0:
            continue
        a = 0
        while a < M:
            u = oracle.sdcp_uniform(2024, bytes(sess[b]["id"]), 5, a + 1, 0)
            if not u < min(1.0, o["p_tok"][b, a] / o["q_tok"][b, a]):
                break
            a += 1
        assert o["accepted_len"][b] == a
    # a different round changes the draws somewhere
    sess2 = oracle.make_sdcp_sessions(B, seed=2024, round_=6)
    o2 = oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"], 0, 0,
                       sdcp_sessions=sess2)
    assert not np.array_equal(o["out_tokens"], o2["out_tokens"])


def test_verify_sdcp_additional_token_uses_purpose_1():
    """Sec. 6.4: the token after the accepted run comes from the purpose-1
    value at position a + 1 -- from norm(max(0, p - q)) after a rejection,
    from p when every drafted token was accepted."""
    rng = np.random.default_rng(13)
    h = _small_batch(rng, B=40)
    B, M = h["tokens"].shape
    sess = oracle.make_sdcp_sessions(B, seed=77, round_=3)
    o = oracle.verify(h["target"], h["draft"], h["tokens"], h["m"], h["rule"], h["sampling"], 0, 0,
                      sdcp_sessions=sess)
    seen = {"residual": 0, "bonus": 0}
    for b in range(B):
        a = int(o["accepted_len"][b])
        if h["rule"][b] != 2 or a < 0:
            continue
        u = oracle.sdcp_uniform(77, bytes(sess[b]["id"]), 3, a + 1, 1)
        _, p, _ = oracle.profile(h["target"][b, a], 900, 0, 950)
        if a < M:
            _, q, _ = oracle.profile(h["draft"][b, a], 900, 0, 950)
            want, _ = oracle.residual_pick(p, q, u)
            seen["residual"] += 1
        else:
            want, _ = oracle.inverse_cdf(p, u)
            seen["bonus"] += 1
        assert o["out_tokens"][b, a] == want
    assert seen["residual"] > 3 and seen["bonus"] > 0
