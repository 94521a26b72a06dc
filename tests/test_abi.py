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
    assert {"sv_verify", "sv_verify_sdcp", "sv_verify_qrows", "sv_workspace_bytes", "sv_strerror",
            "sv_status_str", "sv_version"} <= names


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


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "token_sampling_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "sv_oracle" not in text and "ov_verify" not in text, path
