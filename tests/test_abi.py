"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function declared in include/*.h, and
reject bad call-level arguments on the host before enqueuing anything.
"""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for mt in re.finditer(r"\b(sv_[a-z_0-9]+)\s*\(", text):
            names.add(mt.group(1))
    return names


@pytest.fixture(scope="module")
def svlib():
    import token_sampling_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        from token_sampling_amd import build
        build.build()
    return sv


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"sv_verify", "sv_verify_sdcp", "sv_verify_qrows", "sv_verify_early", "sv_commit",
            "sv_prefix_digest",
            "sv_contract_digest", "sv_workspace_bytes", "sv_strerror", "sv_status_str",
            "sv_version"} <= names


def test_library_exports_every_declared_symbol(svlib):
    L = ctypes.CDLL(svlib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in include/ but not exported"
    assert set(svlib.EXPORTED) == declared_functions()


def test_version_and_strings(svlib):
    L = svlib.lib()
    assert L.sv_version() == 1
    for code in (0, -1, -2, -3, 12345):
        assert isinstance(svlib.strerror(code), str) and svlib.strerror(code)
    for st in (3, 0, -1, -2, -3, -4, -5, -99):
        assert svlib.status_str(st)


def test_workspace_bytes_bounds(svlib):
    assert svlib.workspace_bytes(1, 1, 1) > 0
    assert svlib.workspace_bytes(1024, 64, 129280) > 0
    assert svlib.workspace_bytes(0, 4, 100) == 0
    assert svlib.workspace_bytes(4, 0, 100) == 0
    assert svlib.workspace_bytes(4, 65, 100) == 0
    assert svlib.workspace_bytes(4, 4, 0) == 0
    assert svlib.workspace_bytes(4, 4, (1 << 24) + 1) == 0
    # grows with the batch
    assert svlib.workspace_bytes(512, 8, 1000) > svlib.workspace_bytes(256, 8, 1000)
    # SV_B_MAX = 2^21 sessions, SV_SLOTS_MAX = 2^25 row slots B * (2M + 1)
    assert svlib.workspace_bytes(1 << 21, 1, 10) > 0
    assert svlib.workspace_bytes((1 << 21) + 1, 1, 10) == 0
    assert svlib.workspace_bytes(1 << 19, 31, 10) > 0  # 2^19 * 63 slots
    assert svlib.workspace_bytes(1 << 19, 32, 10) == 0  # 2^19 * 65 slots


def test_verify_rejects_bad_arguments_on_the_host(svlib):
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    ws = svlib.workspace_bytes(2, 2, 10)

    def call(target=fake, tokens=fake, m=fake, rule=fake, smp=fake, B=2, M=2, V=10, dtype=0,
             acc=fake, out=fake, wsp=fake, wsb=ws):
        return L.sv_verify(target, None, dtype, tokens, m, rule, smp, B, M, V, 0, 1, acc, out,
                           wsp, wsb, None, None)

    assert call(target=None) == svlib.ERR_ARG
    assert call(tokens=None) == svlib.ERR_ARG
    assert call(m=None) == svlib.ERR_ARG
    assert call(rule=None) == svlib.ERR_ARG
    assert call(smp=None) == svlib.ERR_ARG
    assert call(acc=None) == svlib.ERR_ARG
    assert call(out=None) == svlib.ERR_ARG
    assert call(wsp=None) == svlib.ERR_ARG
    assert call(B=0) == svlib.ERR_ARG
    assert call(M=0) == svlib.ERR_ARG
    assert call(M=65) == svlib.ERR_ARG
    assert call(V=0) == svlib.ERR_ARG
    assert call(dtype=7) == svlib.ERR_ARG
    assert call(wsb=ws - 1) == svlib.ERR_WORKSPACE


def test_sdcp_session_record_layout(svlib):
    """sv_sdcp_session: id[16] at 0, seed at 16, round at 24, reserved at 28."""
    d = svlib.SDCP_SESSION_DTYPE
    assert d.itemsize == 32
    assert [d.fields[n][1] for n in ("session_id", "seed", "round", "reserved")] == [0, 16, 24, 28]
    text = open(os.path.join(ROOT, "include", "specverify.h")).read()
    body = re.search(r"typedef struct sv_sdcp_session \{(.*?)\} sv_sdcp_session;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(u?int\d+_t)\s+(\w+)(\[\d+\])?;", body)
    assert fields == [("uint8_t", "session_id", "[16]"), ("uint64_t", "seed", ""),
                      ("uint32_t", "round", ""), ("uint32_t", "reserved", "")]


def test_verify_sdcp_rejects_bad_arguments_on_the_host(svlib):
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    ws = svlib.workspace_bytes(2, 2, 10)

    def call(sess=fake, target=fake, B=2, M=2, wsb=ws):
        return L.sv_verify_sdcp(target, None, 0, fake, fake, fake, fake, sess, B, M, 10, fake,
                                fake, fake, wsb, None, None)

    assert call(sess=None) == svlib.ERR_ARG
    assert call(target=None) == svlib.ERR_ARG
    assert call(B=0) == svlib.ERR_ARG
    assert call(M=65) == svlib.ERR_ARG
    assert call(wsb=ws - 1) == svlib.ERR_WORKSPACE


def test_verify_qrows_rejects_bad_arguments_on_the_host(svlib):
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    ws = svlib.workspace_bytes(2, 2, 10)

    def call(target=fake, tokens=fake, dtype=0, B=2, M=2, V=10, wsb=ws, wsp=fake):
        # q_rows and sessions may be NULL; no kernel is reached in these calls
        return L.sv_verify_qrows(target, dtype, None, tokens, fake, fake, fake, None, B, M, V, 0,
                                 1, fake, fake, wsp, wsb, None, None)

    assert call(target=None) == svlib.ERR_ARG
    assert call(tokens=None) == svlib.ERR_ARG
    assert call(wsp=None) == svlib.ERR_ARG
    assert call(dtype=3) == svlib.ERR_ARG
    assert call(B=0) == svlib.ERR_ARG
    assert call(M=65) == svlib.ERR_ARG
    assert call(V=0) == svlib.ERR_ARG
    assert call(wsb=ws - 1) == svlib.ERR_WORKSPACE


def test_verify_early_rejects_bad_arguments_on_the_host(svlib):
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    ws = svlib.workspace_bytes(2, 2, 10)

    def call(target=fake, draft=None, qrows=None, window0=1, B=2, M=2, V=10, wsb=ws, wsp=fake):
        return L.sv_verify_early(target, draft, qrows, 0, fake, fake, fake, fake, None, B, M, V,
                                 0, 1, window0, fake, fake, wsp, wsb, None, None)

    assert call(window0=0) == svlib.ERR_ARG
    assert call(window0=66) == svlib.ERR_ARG
    assert call(draft=fake, qrows=fake) == svlib.ERR_ARG  # one draft source at most
    assert call(target=None) == svlib.ERR_ARG
    assert call(wsp=None) == svlib.ERR_ARG
    assert call(B=0) == svlib.ERR_ARG
    assert call(M=65) == svlib.ERR_ARG
    assert call(V=0) == svlib.ERR_ARG
    assert call(wsb=ws - 1) == svlib.ERR_WORKSPACE
    assert call(window0=65, wsb=ws - 1) == svlib.ERR_WORKSPACE


def header_struct_fields(name):
    text = open(os.path.join(ROOT, "include", "specverify.h")).read()
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return re.findall(r"(u?int\d+_t)\s+([\w, ]+?)(\[\w+\])?;", body)


def test_commit_record_layouts(svlib):
    assert svlib.CONTRACT_DTYPE.itemsize == 64 and svlib.STATE_DTYPE.itemsize == 64
    assert header_struct_fields("sv_contract") == [
        ("uint32_t", "m_max", ""), ("uint32_t", "max_new", ""), ("uint32_t", "low_rounds", ""),
        ("uint32_t", "low_ratio", ""), ("uint32_t", "n_stop", ""), ("int32_t", "stop", "[SV_STOP_MAX]"),
        ("uint32_t", "n_fallback", ""), ("uint8_t", "fallback", "[SV_FALLBACK_MAX]")]
    assert header_struct_fields("sv_session_state") == [
        ("uint8_t", "digest", "[32]"), ("uint32_t", "n", ""), ("uint32_t", "m_cap", ""),
        ("uint32_t", "c, g, j", ""), ("uint32_t", "reserved", "[3]")]
    d = svlib.CONTRACT_DTYPE
    assert [d.fields[f][1] for f in ("m_max", "n_stop", "stop", "n_fallback", "fallback")] == \
        [0, 16, 20, 52, 56]
    d = svlib.STATE_DTYPE
    assert [d.fields[f][1] for f in ("digest", "n", "m_cap", "c", "g", "j")] == \
        [0, 32, 36, 40, 44, 48]


def test_host_digests_reproduce_appendix_a(svlib):
    """The library's host SHA-256 (sv_contract_digest, sv_prefix_digest) against
    the contract digest and d[0] printed in SDCP Appendix A."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "sdcp_appendix_a_digests.json")))
    cd = svlib.contract_digest(bytes.fromhex(g["contract_cbor_hex"]))
    assert cd.hex() == g["contract_digest"]
    assert svlib.prefix_digest(cd, g["prompt"]).hex() == g["d"][0]
    import hashlib
    for n in (0, 1, 55, 56, 63, 64, 119, 120, 1000):
        msg = bytes((3 * i) & 0xFF for i in range(n))
        assert svlib.contract_digest(msg) == hashlib.sha256(b"SDCP-CONTRACT-1\x00" + msg).digest()


def test_commit_rejects_bad_arguments_on_the_host(svlib):
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first

    def call(contracts=fake, states=fake, B=3, M=4, emitted=fake):
        return L.sv_commit(contracts, states, fake, fake, fake, None, B, M, emitted, fake, None)

    assert call(contracts=None) == svlib.ERR_ARG
    assert call(states=None) == svlib.ERR_ARG
    assert call(emitted=None) == svlib.ERR_ARG
    assert call(B=0) == svlib.ERR_ARG
    assert call(M=0) == svlib.ERR_ARG
    assert call(M=65) == svlib.ERR_ARG
    assert L.sv_prefix_digest(None, None, 0, ctypes.create_string_buffer(32)) == svlib.ERR_ARG
    assert L.sv_contract_digest(b"", 0, None) == svlib.ERR_ARG


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "token_sampling_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "sv_oracle" not in text and "ov_verify" not in text, path


def test_noalloc_refuses_on_the_host(svlib):
    """sv_verify_noalloc refuses sizes beyond its device array, and bad sizes,
    before any device call."""
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    B, M, V = 1 << 20, 8, 1 << 20
    assert svlib.workspace_bytes(B, M, V) > (128 << 20)
    assert L.sv_verify_noalloc(fake, fake, 0, fake, fake, fake, fake, B, M, V, 0, 1, fake, fake,
                               None, None) == svlib.ERR_WORKSPACE
    assert L.sv_verify_noalloc(fake, fake, 0, fake, fake, fake, fake, 0, M, V, 0, 1, fake, fake,
                               None, None) == svlib.ERR_ARG
    assert L.sv_verify_noalloc(fake, fake, 7, fake, fake, fake, fake, 4, M, 100, 0, 1, fake, fake,
                               None, None) == svlib.ERR_ARG


def test_verify_commit_refuses_on_the_host(svlib):
    """sv_verify_commit refuses a null commit struct or a null member (other
    than self_decode_ok), and bad sizes, before any device call."""
    L = svlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    B, M, V = 4, 3, 100
    ws = svlib.workspace_bytes(B, M, V)

    def call(cio, B=B, dtype=0):
        return L.sv_verify_commit(fake, fake, dtype, fake, fake, fake, fake, None, B, M, V, 0, 1,
                                  fake, fake, cio, fake, ws, None, None)

    assert call(None) == svlib.ERR_ARG
    full = dict(contracts=0x1000, states=0x1000, self_decode_ok=None, emitted_len=0x1000,
                action=0x1000)
    for k in ("contracts", "states", "emitted_len", "action"):
        io = svlib._CommitIO(**{**full, k: None})
        assert call(ctypes.byref(io)) == svlib.ERR_ARG, k
    io = svlib._CommitIO(**full)
    assert call(ctypes.byref(io), B=0) == svlib.ERR_ARG
    assert call(ctypes.byref(io), dtype=7) == svlib.ERR_ARG
    # the drafted tokens' links live in the workspace: B * M * 32 bytes of it
    assert svlib.workspace_bytes(256, 8, 1000) - svlib.workspace_bytes(256, 7, 1000) >= 256 * 32
