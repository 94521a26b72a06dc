"""ctypes wrapper around the plain-C oracle (``oracle/sv_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` are the only
callers.  The product path (``token_sampling_amd``) never imports this module.

The oracle computes, per session and in IEEE binary64, the acceptance step of
the SDCP Internet-Draft ("Speculative Decoding Coordination Protocol (SDCP) for
Distributed Inference with Multi-Level Caches"), Sec. 4.1 (sampling profile)
and Sec. 6.4 (Rule 1 greedy, Rule 2 speculative sampling), with uniforms from
Philox4x64-10 (Salmon et al., SC'11).  See the header of ``sv_oracle.c`` for
every reading taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "libsv_oracle.so")

BF16 = 0
FP32 = 1
RULE_GREEDY = 1
RULE_SPECULATIVE = 2
RULE_RELAXED = 192  # private use: accept while p_i(x_i) > 0
S_BAD_PROPOSAL = -1
S_LIMIT = -2
S_Q_UNAVAILABLE = -3
S_BAD_PROFILE = -4
S_BAD_LOGITS = -5

SAMPLING_DTYPE = np.dtype(
    [
        ("temperature_milli", "<u4"),
        ("top_k", "<u4"),
        ("top_p_milli", "<u4"),
        ("reserved", "<u4"),
        ("session_key", "<u8"),
    ],
    align=True,
)
assert SAMPLING_DTYPE.itemsize == 24


class _Sampling(ctypes.Structure):
    _fields_ = [
        ("temperature_milli", ctypes.c_uint32),
        ("top_k", ctypes.c_uint32),
        ("top_p_milli", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("session_key", ctypes.c_uint64),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libsv_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-shared", "-fPIC",
             "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        dp = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.ov_philox4x64_10.argtypes = [u64p, u64p, u64p]
        L.ov_philox4x64_10.restype = None
        L.ov_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                 ctypes.c_uint32, ctypes.c_int]
        L.ov_uniform.restype = ctypes.c_double
        L.ov_profile_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(_Sampling), dp, dp]
        L.ov_profile_row.restype = ctypes.c_int
        L.ov_inverse_cdf.argtypes = [dp, ctypes.c_int, ctypes.c_double, dp]
        L.ov_inverse_cdf.restype = ctypes.c_int
        L.ov_residual_pick.argtypes = [dp, dp, ctypes.c_int, ctypes.c_double, dp]
        L.ov_residual_pick.restype = ctypes.c_int
        L.ov_verify.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, i32p, i32p, i32p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_uint64, ctypes.c_uint32, i32p, i32p, dp, dp, dp, dp, dp, dp,
        ]
        L.ov_verify.restype = ctypes.c_int
        L.ov_verify_sdcp.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, i32p, i32p, i32p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            i32p, i32p, dp, dp, dp, dp, dp, dp,
        ]
        L.ov_verify_sdcp.restype = ctypes.c_int
        L.ov_verify_qrows.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, i32p, i32p, i32p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_uint64, ctypes.c_uint32, i32p, i32p, dp, dp, dp, dp, dp,
        ]
        L.ov_verify_qrows.restype = ctypes.c_int
        L.ov_verify_early.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, i32p, i32p, i32p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_uint64, ctypes.c_uint32, i32p, i32p, dp, dp, dp, dp, dp, dp,
        ]
        L.ov_verify_early.restype = ctypes.c_int
        L.ov_commit.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i32p, i32p, i32p,
                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, i32p, i32p]
        L.ov_commit.restype = ctypes.c_int
        L.ov_prefix_digest.argtypes = [ctypes.c_char_p, i32p, ctypes.c_uint32, ctypes.c_char_p]
        L.ov_prefix_digest.restype = None
        L.ov_contract_digest.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p]
        L.ov_contract_digest.restype = None
        L.ov_sha256.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p]
        L.ov_sha256.restype = None
        L.ov_hmac_sha256.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p,
                                     ctypes.c_size_t, ctypes.c_char_p]
        L.ov_hmac_sha256.restype = None
        L.ov_sdcp_uniform.argtypes = [ctypes.c_uint64, ctypes.c_char_p, ctypes.c_uint32,
                                      ctypes.c_uint32, ctypes.c_int]
        L.ov_sdcp_uniform.restype = ctypes.c_double
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------- generator
def philox4x64_10(counter, key):
    """One Philox4x64-10 block: 4 x uint64 counter, 2 x uint64 key -> 4 x uint64."""
    c = np.asarray(counter, dtype=np.uint64).copy()
    k = np.asarray(key, dtype=np.uint64).copy()
    o = np.zeros(4, dtype=np.uint64)
    lib().ov_philox4x64_10(_ptr(c, ctypes.c_uint64), _ptr(k, ctypes.c_uint64),
                           _ptr(o, ctypes.c_uint64))
    return o


def uniform(seed: int, session_key: int, round_: int, i: int, purpose: int) -> float:
    """The verifier's uniform for (seed, session, round, position i, purpose)."""
    return lib().ov_uniform(seed, session_key, round_, i, purpose)


# ------------------------------------------------------------------ profile
def _as_row(row):
    row = np.ascontiguousarray(row)
    if row.dtype == np.uint16:
        return row, BF16
    if row.dtype == np.float32:
        return row, FP32
    raise TypeError("rows are bf16 bits (uint16) or float32")


def profile(row, temperature_milli=1000, top_k=0, top_p_milli=1000):
    """Return (status, prob[V] float64, delta_topp) for one logits row."""
    row, dt = _as_row(row)
    V = row.shape[-1]
    s = _Sampling(temperature_milli, top_k, top_p_milli, 0, 0)
    prob = np.zeros(V, dtype=np.float64)
    d = np.zeros(1, dtype=np.float64)
    st = lib().ov_profile_row(row.ctypes.data, dt, V, ctypes.byref(s),
                              _ptr(prob, ctypes.c_double), _ptr(d, ctypes.c_double))
    return st, prob, float(d[0])


def inverse_cdf(w, u):
    """Return (token, delta) for the inverse CDF of weights w (ascending ids)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    d = np.zeros(1, dtype=np.float64)
    y = lib().ov_inverse_cdf(_ptr(w, ctypes.c_double), w.shape[0], u, _ptr(d, ctypes.c_double))
    return y, float(d[0])


def residual_pick(p, q, u):
    """Return (token, delta): the draw from norm(max(0, p - q)) (p if that has no mass)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    d = np.zeros(1, dtype=np.float64)
    y = lib().ov_residual_pick(_ptr(p, ctypes.c_double), _ptr(q, ctypes.c_double), p.shape[0],
                               u, _ptr(d, ctypes.c_double))
    return y, float(d[0])


# ------------------------------------------------------------- batched step
# SDCP per-session inputs of the verifier's uniforms (Sec. 6.4): the 16-octet
# session id, the profile's seed and the round (32 bytes, 8-aligned).
SDCP_SESSION_DTYPE = np.dtype(
    [("id", np.uint8, (16,)), ("seed", np.uint64), ("round", np.uint32), ("reserved", np.uint32)],
    align=True)
assert SDCP_SESSION_DTYPE.itemsize == 32


def sha256(msg: bytes) -> bytes:
    """SHA-256 (FIPS 180-4) of msg, by the oracle's own implementation."""
    out = ctypes.create_string_buffer(32)
    lib().ov_sha256(msg, len(msg), out)
    return out.raw


def hmac_sha256(key: bytes, msg: bytes) -> bytes:
    """HMAC-SHA-256 (RFC 2104) by the oracle's own implementation."""
    out = ctypes.create_string_buffer(32)
    lib().ov_hmac_sha256(key, len(key), msg, len(msg), out)
    return out.raw


def sdcp_uniform(seed: int, session: bytes, round_: int, i: int, purpose: int) -> float:
    """SDCP Sec. 6.4 verifier value for position i (purpose 0 or 1)."""
    assert len(session) == 16
    return lib().ov_sdcp_uniform(seed, session, round_, i, purpose)


def make_sdcp_sessions(B, seed=0, round_=1, ids=None):
    """SDCP session records: ids [B, 16] uint8 (default: b in the last 8
    octets, big-endian), one seed and round for all (or arrays [B])."""
    s = np.zeros(B, dtype=SDCP_SESSION_DTYPE)
    if ids is None:
        for b in range(B):
            s[b]["id"][8:] = np.frombuffer(int(b).to_bytes(8, "big"), dtype=np.uint8)
    else:
        s["id"] = np.asarray(ids, dtype=np.uint8).reshape(B, 16)
    s["seed"] = seed
    s["round"] = round_
    return s


def make_sampling(B, temperature_milli=1000, top_k=0, top_p_milli=1000, session_key=None):
    s = np.zeros(B, dtype=SAMPLING_DTYPE)
    s["temperature_milli"] = temperature_milli
    s["top_k"] = top_k
    s["top_p_milli"] = top_p_milli
    s["session_key"] = np.arange(B, dtype=np.uint64) if session_key is None else session_key
    return s


def verify(target, draft, tokens, m, rule, sampling, seed, round_, diagnostics=True,
           sdcp_sessions=None, q_rows=None, early=False):
    """Run the oracle over a batch.

    target: [B, M+1, V] uint16 (bf16 bits) or float32; draft: [B, M, V] of the
    same dtype, or None.  tokens [B, M] int32, m [B] int32, rule [B] int32,
    sampling [B] of ``SAMPLING_DTYPE``.  Returns a dict with accepted_len,
    out_tokens, p_tok, q_tok and (if diagnostics) d_acc, d_topp_t, d_topp_d,
    d_cdf.  With sdcp_sessions ([B] of ``SDCP_SESSION_DTYPE``) the uniforms are
    SDCP's HMAC-SHA-256 values and seed, round_ are ignored.  With q_rows
    ([B, M, V] float32 probabilities, SDCP's q_rows) the draft distributions
    are those rows and draft must be None; d_topp_d is then not computed.
    With early=True positions are examined in order and each row is read only
    when its position is reached (``ov_verify_early``): a problem in a row
    after the deciding position changes nothing, and the probes and
    diagnostics hold values only up to that position.
    """
    target = np.ascontiguousarray(target)
    _, dt = _as_row(target[..., :1].reshape(-1)[:1]) if target.size else (None, BF16)
    B, M1, V = target.shape
    M = M1 - 1
    if draft is not None:
        draft = np.ascontiguousarray(draft)
        assert draft.dtype == target.dtype and draft.shape == (B, M, V)
    if q_rows is not None:
        assert draft is None, "give draft logits or q_rows, not both"
        q_rows = np.ascontiguousarray(q_rows, dtype=np.float32)
        assert q_rows.shape == (B, M, V)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, M)
    m = np.ascontiguousarray(m, dtype=np.int32).reshape(B)
    rule = np.ascontiguousarray(rule, dtype=np.int32).reshape(B)
    sampling = np.ascontiguousarray(sampling, dtype=SAMPLING_DTYPE).reshape(B)
    out = {
        "accepted_len": np.zeros(B, dtype=np.int32),
        "out_tokens": np.zeros((B, M + 1), dtype=np.int32),
        "p_tok": np.zeros((B, M), dtype=np.float64),
        "q_tok": np.zeros((B, M), dtype=np.float64),
    }
    if diagnostics:
        out["d_acc"] = np.zeros((B, M), dtype=np.float64)
        out["d_topp_t"] = np.zeros((B, M + 1), dtype=np.float64)
        out["d_topp_d"] = np.zeros((B, M), dtype=np.float64)
        out["d_cdf"] = np.zeros(B, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)

    def opt(name):
        return _ptr(out[name], ctypes.c_double) if name in out else ctypes.cast(None, dp)

    outs = (_ptr(out["accepted_len"], ctypes.c_int32), _ptr(out["out_tokens"], ctypes.c_int32),
            opt("p_tok"), opt("q_tok"), opt("d_acc"), opt("d_topp_t"), opt("d_topp_d"),
            opt("d_cdf"))
    common = (target.ctypes.data, None if draft is None else draft.ctypes.data, dt,
              _ptr(tokens, ctypes.c_int32), _ptr(m, ctypes.c_int32), _ptr(rule, ctypes.c_int32),
              sampling.ctypes.data)
    sess = None
    if sdcp_sessions is not None:
        sess = np.ascontiguousarray(sdcp_sessions, dtype=SDCP_SESSION_DTYPE).reshape(B)
    if early:
        rc = lib().ov_verify_early(target.ctypes.data, common[1],
                                   None if q_rows is None else q_rows.ctypes.data, *common[2:],
                                   None if sess is None else sess.ctypes.data, B, M, V, seed,
                                   round_, *outs)
    elif q_rows is not None:
        no_d_topp_d = outs[:6] + outs[7:]
        rc = lib().ov_verify_qrows(target.ctypes.data, dt, q_rows.ctypes.data, *common[3:],
                                   None if sess is None else sess.ctypes.data, B, M, V, seed,
                                   round_, *no_d_topp_d)
        if "d_topp_d" in out:
            out["d_topp_d"][:] = np.inf
    elif sdcp_sessions is None:
        rc = lib().ov_verify(*common, B, M, V, seed, round_, *outs)
    else:
        sess = np.ascontiguousarray(sdcp_sessions, dtype=SDCP_SESSION_DTYPE).reshape(B)
        rc = lib().ov_verify_sdcp(*common, sess.ctypes.data, B, M, V, *outs)
    if rc != 0:
        raise ValueError(f"oracle rejected the call (code {rc})")
    return out


# ------------------------------------------------------------- commit step
# SDCP Sec. 6.5.2 actions
ACT_CONTINUE, ACT_REDUCE, ACT_SWITCH, ACT_SELF_DECODE, ACT_FINISH, ACT_FAIL = range(6)

CONTRACT_DTYPE = np.dtype(
    [("m_max", "<u4"), ("max_new", "<u4"), ("low_rounds", "<u4"), ("low_ratio", "<u4"),
     ("n_stop", "<u4"), ("stop", "<i4", (8,)), ("n_fallback", "<u4"), ("fallback", "u1", (8,))],
    align=True)
assert CONTRACT_DTYPE.itemsize == 64

STATE_DTYPE = np.dtype(
    [("digest", "u1", (32,)), ("n", "<u4"), ("m_cap", "<u4"), ("c", "<u4"), ("g", "<u4"),
     ("j", "<u4"), ("reserved", "<u4", (3,))],
    align=True)
assert STATE_DTYPE.itemsize == 64


def make_contracts(B, m_max=8, max_new=256, low_rounds=3, low_ratio=0, stop=(2,),
                   fallback=(ACT_REDUCE, ACT_SWITCH, ACT_SELF_DECODE, ACT_FAIL)):
    c = np.zeros(B, dtype=CONTRACT_DTYPE)
    c["m_max"], c["max_new"], c["low_rounds"], c["low_ratio"] = m_max, max_new, low_rounds, low_ratio
    c["n_stop"] = len(stop)
    c["stop"][:, :len(stop)] = stop
    c["n_fallback"] = len(fallback)
    c["fallback"][:, :len(fallback)] = fallback
    return c


def make_states(B, digest=b"\0" * 32, n=0, m_cap=8):
    s = np.zeros(B, dtype=STATE_DTYPE)
    s["digest"] = np.frombuffer(bytes(digest), dtype=np.uint8)
    s["n"], s["m_cap"] = n, m_cap
    return s


def prefix_digest(contract_digest: bytes, prompt) -> bytes:
    """d[0] of SDCP Sec. 4.2."""
    p = np.ascontiguousarray(prompt, dtype=np.int32)
    out = ctypes.create_string_buffer(32)
    lib().ov_prefix_digest(bytes(contract_digest), _ptr(p, ctypes.c_int32), p.shape[0], out)
    return out.raw


def contract_digest(cbor: bytes) -> bytes:
    """contract_digest of SDCP Sec. 4.1 over a deterministic CBOR encoding."""
    out = ctypes.create_string_buffer(32)
    lib().ov_contract_digest(bytes(cbor), len(cbor), out)
    return out.raw


def commit(contracts, states, m, accepted_len, out_tokens, self_decode_ok=None):
    """The commit step (SDCP Sec. 6.3 steps 6-8, 6.5) for one round.  states is
    updated in place; returns (out_tokens truncated, emitted_len, action)."""
    contracts = np.ascontiguousarray(contracts, dtype=CONTRACT_DTYPE)
    assert states.dtype == STATE_DTYPE and states.flags["C_CONTIGUOUS"]
    B = states.shape[0]
    out = np.array(out_tokens, dtype=np.int32, copy=True).reshape(B, -1)
    M = out.shape[1] - 1
    m = np.ascontiguousarray(m, dtype=np.int32).reshape(B)
    a = np.ascontiguousarray(accepted_len, dtype=np.int32).reshape(B)
    ok = None if self_decode_ok is None else np.ascontiguousarray(self_decode_ok, dtype=np.uint8)
    emitted = np.zeros(B, dtype=np.int32)
    action = np.zeros(B, dtype=np.int32)
    rc = lib().ov_commit(contracts.ctypes.data, states.ctypes.data, _ptr(m, ctypes.c_int32),
                         _ptr(a, ctypes.c_int32), _ptr(out, ctypes.c_int32),
                         None if ok is None else ok.ctypes.data, B, M,
                         _ptr(emitted, ctypes.c_int32), _ptr(action, ctypes.c_int32))
    if rc != 0:
        raise ValueError(f"oracle rejected the call (code {rc})")
    return out, emitted, action


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) and return the bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    nan = np.isnan(x)
    bits = (rounded >> np.uint32(16)).astype(np.uint16)
    bits[nan] = np.uint16(0x7FC0)
    return bits


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
