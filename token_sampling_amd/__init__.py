"""token_sampling_amd -- Python binding of libspecverify, the MI355X (gfx950)
verifier acceptance step for speculative decoding.

This module only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates outputs and the workspace with torch, and calls the C ABI
declared in ``include/specverify.h`` on the current torch stream.  Every step
of the computation runs in the HIP kernels of ``libspecverify.so``; there is
no CPU or PyTorch fallback, and the calls raise if the library is missing.

The operation is the acceptance step of the SDCP Internet-Draft ("Speculative
Decoding Coordination Protocol (SDCP) for Distributed Inference with
Multi-Level Caches"), Sec. 4.1 (sampling profile) and Sec. 6.4 (Rule 1 greedy,
Rule 2 speculative sampling).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

BF16 = 0
FP32 = 1
RULE_GREEDY = 1
RULE_SPECULATIVE = 2
RULE_RELAXED = 192  # private use: accept while p_i(x_i) > 0
OK = 0
ERR_ARG = -1
ERR_DEVICE = -2
ERR_WORKSPACE = -3
S_BAD_PROPOSAL = -1
S_LIMIT = -2
S_Q_UNAVAILABLE = -3
S_BAD_PROFILE = -4
S_BAD_LOGITS = -5

SAMPLING_DTYPE = np.dtype(
    [("temperature_milli", "<u4"), ("top_k", "<u4"), ("top_p_milli", "<u4"),
     ("reserved", "<u4"), ("session_key", "<u8")],
    align=True,
)
# SDCP Sec. 6.4 inputs of the verifier values: 16-octet session id, the
# profile's seed, the round (32 bytes, 8-aligned; sv_sdcp_session).
SDCP_SESSION_DTYPE = np.dtype(
    [("session_id", np.uint8, (16,)), ("seed", "<u8"), ("round", "<u4"), ("reserved", "<u4")],
    align=True,
)
# SDCP Sec. 6.5.2 actions and the commit step's records (sv_contract,
# sv_session_state, 64 bytes each).
ACT_CONTINUE, ACT_REDUCE, ACT_SWITCH, ACT_SELF_DECODE, ACT_FINISH, ACT_FAIL = range(6)
CONTRACT_DTYPE = np.dtype(
    [("m_max", "<u4"), ("max_new", "<u4"), ("low_rounds", "<u4"), ("low_ratio", "<u4"),
     ("n_stop", "<u4"), ("stop", "<i4", (8,)), ("n_fallback", "<u4"), ("fallback", "u1", (8,))],
    align=True,
)
STATE_DTYPE = np.dtype(
    [("digest", "u1", (32,)), ("n", "<u4"), ("m_cap", "<u4"), ("c", "<u4"), ("g", "<u4"),
     ("j", "<u4"), ("reserved", "<u4", (3,))],
    align=True,
)
EXPORTED = ("sv_workspace_bytes", "sv_verify", "sv_verify_sdcp", "sv_verify_qrows",
            "sv_verify_early", "sv_commit",
            "sv_prefix_digest", "sv_contract_digest", "sv_strerror", "sv_status_str",
            "sv_version", "sv_bench_row_events", "sv_verify_noalloc", "sv_verify_commit")


class SvError(RuntimeError):
    pass


class _Probe(ctypes.Structure):
    _fields_ = [("p_tok", ctypes.c_void_p), ("q_tok", ctypes.c_void_p)]


class _CommitIO(ctypes.Structure):
    _fields_ = [("contracts", ctypes.c_void_p), ("states", ctypes.c_void_p),
                ("self_decode_ok", ctypes.c_void_p), ("emitted_len", ctypes.c_void_p),
                ("action", ctypes.c_void_p)]


class HipEvent:
    """A raw hipEvent_t (for the benchmark hook's row-kernel timing slots)."""

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = h
        self._destroy = HipEvent._hip.hipEventDestroy  # kept for interpreter shutdown
        self.handle = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise SvError(f"hipEventCreate failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        HipEvent._hip.hipEventSynchronize(end.handle)
        ms = ctypes.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise SvError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self.handle:
            self._destroy(self.handle)


_lib = None


def lib():
    """Load libspecverify.so (raises SvError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SvError(f"{LIB_PATH} is missing: run token_sampling_amd.build.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.sv_workspace_bytes.argtypes = [ctypes.c_int32] * 3
        L.sv_workspace_bytes.restype = ctypes.c_size_t
        L.sv_verify.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify.restype = ctypes.c_int
        L.sv_verify_sdcp.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify_sdcp.restype = ctypes.c_int
        L.sv_verify_qrows.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify_qrows.restype = ctypes.c_int
        L.sv_verify_early.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify_early.restype = ctypes.c_int
        L.sv_commit.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_void_p, ctypes.c_void_p,
                                                         ctypes.c_void_p]
        L.sv_commit.restype = ctypes.c_int
        L.sv_prefix_digest.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.c_char_p]
        L.sv_prefix_digest.restype = ctypes.c_int
        L.sv_contract_digest.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p]
        L.sv_contract_digest.restype = ctypes.c_int
        L.sv_strerror.argtypes = [ctypes.c_int]
        L.sv_strerror.restype = ctypes.c_char_p
        L.sv_status_str.argtypes = [ctypes.c_int]
        L.sv_status_str.restype = ctypes.c_char_p
        L.sv_version.argtypes = []
        L.sv_version.restype = ctypes.c_int
        L.sv_bench_row_events.argtypes = [ctypes.c_void_p] * 3
        L.sv_bench_row_events.restype = ctypes.c_int
        L.sv_verify_noalloc.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify_noalloc.restype = ctypes.c_int
        L.sv_verify_commit.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_CommitIO),
            ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(_Probe), ctypes.c_void_p,
        ]
        L.sv_verify_commit.restype = ctypes.c_int
        _lib = L
    return _lib


def workspace_bytes(B: int, M: int, V: int) -> int:
    return int(lib().sv_workspace_bytes(B, M, V))


def strerror(code: int) -> str:
    return lib().sv_strerror(code).decode()


def status_str(status: int) -> str:
    return lib().sv_status_str(status).decode()


def make_sampling(B, temperature_milli=1000, top_k=0, top_p_milli=1000, session_key=None,
                  device="cuda"):
    """Pack per-session profiles into the [B] x 24-byte device array."""
    import torch

    s = np.zeros(B, dtype=SAMPLING_DTYPE)
    s["temperature_milli"] = temperature_milli
    s["top_k"] = top_k
    s["top_p_milli"] = top_p_milli
    s["session_key"] = np.arange(B, dtype=np.uint64) if session_key is None else session_key
    raw = np.ascontiguousarray(s).view(np.uint8).reshape(B, 24)
    return torch.from_numpy(raw.copy()).to(device)


def make_sdcp_sessions(B, seed, round_, session_ids=None, device="cuda"):
    """Pack per-session SDCP value inputs into the [B] x 32-byte device array.

    seed and round_ are scalars or length-B sequences; session_ids is a
    [B, 16] array of octets (default: b as the last eight octets, big-endian).
    """
    import torch

    s = np.zeros(B, dtype=SDCP_SESSION_DTYPE)
    if session_ids is None:
        ids = np.zeros((B, 16), dtype=np.uint8)
        ids[:, 8:] = np.arange(B, dtype=">u8").view(np.uint8).reshape(B, 8)
    else:
        ids = np.asarray(session_ids, dtype=np.uint8).reshape(B, 16)
    s["session_id"] = ids
    s["seed"] = seed
    s["round"] = round_
    raw = np.ascontiguousarray(s).view(np.uint8).reshape(B, 32)
    return torch.from_numpy(raw.copy()).to(device)


def make_contracts(B, m_max=8, max_new=256, low_rounds=3, low_ratio=0, stop=(),
                   fallback=(ACT_REDUCE, ACT_SWITCH, ACT_SELF_DECODE, ACT_FAIL), device="cuda"):
    """Pack per-session contract members (SDCP Sec. 4.1) into [B, 64] device bytes.
    Every argument is a scalar (or a sequence, for stop and fallback) shared by
    all sessions, or a list of B of them."""
    import torch

    c = np.zeros(B, dtype=CONTRACT_DTYPE)
    c["m_max"], c["max_new"], c["low_rounds"], c["low_ratio"] = m_max, max_new, low_rounds, low_ratio
    per = [stop] * B if len(stop) == 0 or np.isscalar(stop[0]) else stop
    for b, st in enumerate(per):
        c["n_stop"][b] = len(st)
        c["stop"][b, :min(len(st), 8)] = list(st)[:8]
    per = [fallback] * B if len(fallback) == 0 or np.isscalar(fallback[0]) else fallback
    for b, fb in enumerate(per):
        c["n_fallback"][b] = len(fb)
        c["fallback"][b, :min(len(fb), 8)] = list(fb)[:8]
    raw = np.ascontiguousarray(c).view(np.uint8).reshape(B, 64)
    return torch.from_numpy(raw.copy()).to(device)


def make_states(B, digest=b"\0" * 32, n=0, m_cap=8, device="cuda"):
    """Initial per-session states ([B, 64] device bytes): digest d[n] (32 bytes,
    or a [B, 32] array), n committed tokens, m_cap, counters zero."""
    import torch

    s = np.zeros(B, dtype=STATE_DTYPE)
    s["digest"] = np.asarray(np.frombuffer(digest, np.uint8) if isinstance(digest, bytes)
                             else digest, dtype=np.uint8)
    s["n"], s["m_cap"] = n, m_cap
    raw = np.ascontiguousarray(s).view(np.uint8).reshape(B, 64)
    return torch.from_numpy(raw.copy()).to(device)


def states_numpy(states):
    """Host copy of device state records as a STATE_DTYPE array."""
    raw = states.cpu().numpy().astype(np.uint8, copy=False)
    return raw.reshape(-1, 64).copy().view(STATE_DTYPE).reshape(-1)


def prefix_digest(contract_digest: bytes, prompt) -> bytes:
    """d[0] of SDCP Sec. 4.2 (host)."""
    p = np.ascontiguousarray(prompt, dtype=np.int32)
    out = ctypes.create_string_buffer(32)
    rc = lib().sv_prefix_digest(bytes(contract_digest), p.ctypes.data, p.shape[0], out)
    if rc != OK:
        raise SvError(f"sv_prefix_digest failed ({rc})")
    return out.raw


def contract_digest(cbor: bytes) -> bytes:
    """contract_digest of SDCP Sec. 4.1 over a deterministic CBOR encoding (host)."""
    out = ctypes.create_string_buffer(32)
    rc = lib().sv_contract_digest(bytes(cbor), len(cbor), out)
    if rc != OK:
        raise SvError(f"sv_contract_digest failed ({rc})")
    return out.raw


def commit(contracts, states, m, accepted_len, out_tokens, self_decode_ok=None, stream=None,
           out=None):
    """sv_commit on device tensors: contracts [B, 64] and states [B, 64] uint8
    (see make_contracts / make_states), m and accepted_len [B] int32, out_tokens
    [B, M+1] int32 (truncated in place), self_decode_ok [B] uint8 or None.
    Returns dict(emitted_len, action), both [B] int32."""
    import torch

    dev = out_tokens.device
    B, M1 = out_tokens.shape
    for t, name, dt in ((contracts, "contracts", torch.uint8), (states, "states", torch.uint8)):
        _check(t, name, dt, (B, 64), dev)
    _check(m, "m", torch.int32, (B,), dev)
    _check(accepted_len, "accepted_len", torch.int32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, M1), dev)
    if self_decode_ok is not None:
        _check(self_decode_ok, "self_decode_ok", torch.uint8, (B,), dev)
    if out is None:
        out = {"emitted_len": torch.empty(B, dtype=torch.int32, device=dev),
               "action": torch.empty(B, dtype=torch.int32, device=dev)}
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = lib().sv_commit(contracts.data_ptr(), states.data_ptr(), m.data_ptr(),
                         accepted_len.data_ptr(), out_tokens.data_ptr(),
                         None if self_decode_ok is None else self_decode_ok.data_ptr(), B, M1 - 1,
                         out["emitted_len"].data_ptr(), out["action"].data_ptr(),
                         stream.cuda_stream)
    if rc != OK:
        raise SvError(f"sv_commit failed: {strerror(rc)} ({rc})")
    return out


def _check(t, name, dtype, shape, device):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def verify(target, draft, tokens, m, rule, sampling, seed: int, round_: int, probe: bool = False,
           workspace=None, out=None, stream=None, row_events=None, sdcp_sessions=None,
           q_rows=None, early=None, commit=None):
    """sv_verify, sv_verify_sdcp, sv_verify_qrows or sv_verify_early on torch
    tensors (all on one GPU device).

    target [B, M+1, V] bf16/fp32, draft [B, M, V] same dtype or None, tokens
    [B, M] int32, m [B] int32, rule [B] int32, sampling [B, 24] uint8 (see
    make_sampling).  Returns a dict with accepted_len [B] and out_tokens
    [B, M+1] (int32), plus p_tok and q_tok [B, M] float64 if probe.  The call
    is asynchronous on ``stream`` (default: torch's current stream).
    row_events: optional (start, stop) or (start, mid, stop) HipEvents recorded
        around the row kernels, mid between the single-pass kernel and the other
        (the library's benchmark hook, sv_bench_row_events, set for this call).
    sdcp_sessions: optional [B, 32] uint8 device array (see make_sdcp_sessions);
        then the SDCP Sec. 6.4 values are used and seed, round_ are ignored.
    q_rows: optional [B, M, V] float32 draft distributions (SDCP q_rows) in place
        of draft logits (draft must then be None): sv_verify_qrows.
    early: the first window (1..65 positions) of the in-order reading,
        sv_verify_early (with either draft source and either value source); None:
        every row is read.
    commit: optional (contracts, states, self_decode_ok or None), device arrays
        as for commit(): the acceptance step and the commit step in one call,
        sv_verify_commit (draft logits, either value source, every row read);
        the result then also holds emitted_len and action [B] int32, and out_tokens
        is truncated as sv_commit truncates it.
    """
    import torch

    if not (isinstance(target, torch.Tensor) and target.dim() == 3):
        raise ValueError("target must be a [B, M+1, V] tensor")
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    B, M1, V = target.shape
    M = M1 - 1
    if target.dtype == torch.bfloat16:
        dt = BF16
    elif target.dtype == torch.float32:
        dt = FP32
    else:
        raise TypeError("logits must be bfloat16 or float32")
    _check(target, "target", None, None, dev)
    if draft is not None:
        _check(draft, "draft", target.dtype, (B, M, V), dev)
    _check(tokens, "tokens", torch.int32, (B, M), dev)
    _check(m, "m", torch.int32, (B,), dev)
    _check(rule, "rule", torch.int32, (B,), dev)
    _check(sampling, "sampling", None, None, dev)
    if sampling.numel() * sampling.element_size() != 24 * B:
        raise ValueError("sampling must hold B 24-byte records")
    if q_rows is not None:
        if draft is not None:
            raise ValueError("give draft logits or q_rows, not both")
        _check(q_rows, "q_rows", torch.float32, (B, M, V), dev)
    if sdcp_sessions is not None:
        _check(sdcp_sessions, "sdcp_sessions", None, None, dev)
        if sdcp_sessions.numel() * sdcp_sessions.element_size() != 32 * B:
            raise ValueError("sdcp_sessions must hold B 32-byte records")

    cio = None
    if commit is not None:
        if q_rows is not None or early is not None:
            raise ValueError("commit= takes draft logits and reads every row")
        contracts, states, self_ok = commit
        for t, name in ((contracts, "contracts"), (states, "states")):
            _check(t, name, torch.uint8, (B, 64), dev)
        if self_ok is not None:
            _check(self_ok, "self_decode_ok", torch.uint8, (B,), dev)
    need = workspace_bytes(B, M, V)
    if need == 0:
        raise SvError("sizes out of range")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise SvError("workspace too small")
    if out is None:
        out = {
            "accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((B, M + 1), dtype=torch.int32, device=dev),
        }
        if probe:
            out["p_tok"] = torch.empty((B, M), dtype=torch.float64, device=dev)
            out["q_tok"] = torch.empty((B, M), dtype=torch.float64, device=dev)
    if commit is not None:
        for k in ("emitted_len", "action"):
            if k not in out:
                out[k] = torch.empty(B, dtype=torch.int32, device=dev)
        cio = ctypes.byref(_CommitIO(contracts.data_ptr(), states.data_ptr(),
                                     None if self_ok is None else self_ok.data_ptr(),
                                     out["emitted_len"].data_ptr(), out["action"].data_ptr()))
    pr = None
    if "p_tok" in out:
        pr = ctypes.byref(_Probe(out["p_tok"].data_ptr(), out["q_tok"].data_ptr()))
    evs = None
    if row_events is not None:
        evs = ([row_events[0].handle, None, row_events[1].handle] if len(row_events) == 2
               else [e.handle for e in row_events])
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    common = (target.data_ptr(), None if draft is None else draft.data_ptr(), dt,
              tokens.data_ptr(), m.data_ptr(), rule.data_ptr(), sampling.data_ptr())
    tail = (out["accepted_len"].data_ptr(), out["out_tokens"].data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), pr,
            stream.cuda_stream)
    sess = None if sdcp_sessions is None else sdcp_sessions.data_ptr()
    if evs is not None:
        lib().sv_bench_row_events(*evs)
    try:
        if cio is not None:
            name = "sv_verify_commit"
            rc = lib().sv_verify_commit(*common, sess, B, M, V, seed, round_, tail[0], tail[1],
                                        cio, *tail[2:])
        else:
            rc, name = _call(common, tail, target, q_rows, dt, sess, B, M, V, seed, round_,
                             early)
    finally:
        if evs is not None:
            lib().sv_bench_row_events(None, None, None)
    if rc != OK:
        raise SvError(f"{name} failed: {strerror(rc)} ({rc})")
    return out


def _call(common, tail, target, q_rows, dt, sess, B, M, V, seed, round_, early):
    if early is not None:
        name = "sv_verify_early"
        rc = lib().sv_verify_early(target.data_ptr(), common[1],
                                   None if q_rows is None else q_rows.data_ptr(), dt,
                                   *common[3:], sess, B, M, V, seed, round_, int(early), *tail)
    elif q_rows is not None:
        name = "sv_verify_qrows"
        rc = lib().sv_verify_qrows(target.data_ptr(), dt, q_rows.data_ptr(), *common[3:], sess,
                                   B, M, V, seed, round_, *tail)
    elif sess is None:
        name = "sv_verify"
        rc = lib().sv_verify(*common, B, M, V, seed, round_, *tail)
    else:
        name = "sv_verify_sdcp"
        rc = lib().sv_verify_sdcp(*common, sess, B, M, V, *tail)
    return rc, name
