"""C-ABI checks that need no GPU: the library loads, exports every function that
include/gdr.h declares, and rejects bad arguments with the documented codes
before enqueuing anything (all pointers here are fake and never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")
LIB = os.path.join(ROOT, "matrix_memory_rnn_amd", "libgdr.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libgdr.so not built")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdr_\w+)\s*\(", txt, re.M)))


def _codes():
    txt = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(GDR_\w+)\s+(-?\d+)", txt)}


@pytest.fixture(scope="module")
def lib():
    import matrix_memory_rnn_amd as m
    return m.load_library()


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("gdr_chunk_fwd", "gdr_chunk_fwd_ws", "gdr_chunk_workspace_size", "gdr_chunk_intra",
              "gdr_chunk_scan", "gdr_decode_step", "gdr_mlstm_fwd", "gdr_mlstm_fwd_ws",
              "gdr_mlstm_workspace_size", "gdr_status_string", "gdr_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdr_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_symbols_resolve_through_dlopen(lib):
    for n in _declared():
        assert hasattr(lib, n)
    assert lib.gdr_version() == 200


def test_status_strings(lib):
    codes = _codes()
    for name, val in codes.items():
        if name.startswith("GDR_ERR_") or name == "GDR_OK":
            s = lib.gdr_status_string(val).decode()
            assert s and s != "unknown status"
    assert lib.gdr_status_string(12345).decode() == "unknown status"


# fake, 16-byte aligned, well-separated device addresses (never touched)
BASE = 0x7F0000000000
P = [BASE + i * (1 << 32) for i in range(16)]


def _chunk(lib, ptrs=None, B=1, H=2, T=64, dk=16, dv=16, chunk=16, dtype=1, S0=None, S_out=None):
    p = list(P[:7]) if ptrs is None else ptrs
    return lib.gdr_chunk_fwd(p[0], p[1], p[2], p[3], p[4], p[5], S0, p[6], S_out,
                             B, H, T, dk, dv, chunk, dtype, None)


def test_chunk_validation(lib):
    c = _codes()
    assert _chunk(lib, ptrs=[None] + P[1:7]) == c["GDR_ERR_NULL"]
    assert _chunk(lib, T=0) == c["GDR_ERR_SHAPE"]
    assert _chunk(lib, B=0) == c["GDR_ERR_SHAPE"]
    # one head's bytes must stay below 2**31 (32-bit signed offsets in the kernels)
    assert _chunk(lib, T=1 << 23, dk=128, dv=128, chunk=64, dtype=1) == c["GDR_ERR_SHAPE"]
    assert _chunk(lib, T=1 << 22, dk=128, dv=128, chunk=32, dtype=0) == c["GDR_ERR_SHAPE"]
    assert _chunk(lib, dtype=7) == c["GDR_ERR_DTYPE"]
    assert _chunk(lib, dk=48) == c["GDR_ERR_UNSUPPORTED"]
    assert _chunk(lib, dv=256) == c["GDR_ERR_UNSUPPORTED"]
    assert _chunk(lib, chunk=128) == c["GDR_ERR_UNSUPPORTED"]
    assert _chunk(lib, dk=128, dv=128, chunk=64, dtype=0) == c["GDR_ERR_UNSUPPORTED"]
    assert _chunk(lib, dk=64, dv=16, chunk=64, dtype=0) == c["GDR_ERR_UNSUPPORTED"]
    assert _chunk(lib, ptrs=[P[0] + 8] + P[1:7]) == c["GDR_ERR_ALIGN"]
    assert _chunk(lib, S0=P[8] + 4) == c["GDR_ERR_ALIGN"]
    # o overlapping q
    assert _chunk(lib, ptrs=P[:6] + [P[0] + 64]) == c["GDR_ERR_ALIAS"]
    # S_out overlapping (but not equal to) S0
    assert _chunk(lib, S0=P[8], S_out=P[8] + 256) == c["GDR_ERR_ALIAS"]


def _ws_size(lib, B=1, H=2, T=64, dk=16, dv=16, chunk=16, dtype=1):
    n = ctypes.c_size_t(123)
    st = lib.gdr_chunk_workspace_size(B, H, T, dk, dv, chunk, dtype, ctypes.byref(n))
    return st, n.value


def test_workspace_size(lib):
    c = _codes()
    # one record per (b, h, chunk): C*dk (Y) + dv*C (U^T) + C*C (M) + C*dk (Q_pi) + dk*C (K~^T)
    # elements of the input dtype, then dk float32 (pi_C)
    for (B, H, T, dk, dv, C, dt) in ((1, 2, 64, 16, 16, 16, 1), (4, 16, 4096, 128, 128, 64, 1),
                                     (2, 3, 333, 64, 32, 32, 0)):
        es = 2 if dt == 1 else 4
        rec = (3 * C * dk + dv * C + C * C) * es + 4 * dk
        st, n = _ws_size(lib, B, H, T, dk, dv, C, dt)
        assert st == c["GDR_OK"] and n == B * H * ((T + C - 1) // C) * rec
    assert _ws_size(lib, T=0) == (c["GDR_ERR_SHAPE"], 0)
    assert _ws_size(lib, chunk=48)[0] == c["GDR_ERR_UNSUPPORTED"]
    assert lib.gdr_chunk_workspace_size(1, 1, 1, 16, 16, 16, 1, None) == c["GDR_ERR_NULL"]


def test_chunk_ws_validation(lib):
    c = _codes()
    need = _ws_size(lib)[1]

    def f(ws=P[10], nbytes=None, ptrs=None, dtype=1, dk=16, chunk=16):
        p = list(P[:7]) if ptrs is None else ptrs
        return lib.gdr_chunk_fwd_ws(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], None,
                                    1, 2, 64, dk, 16, chunk, dtype, ws, need if nbytes is None else nbytes, None)

    assert f(ws=None) == c["GDR_ERR_NULL"]
    assert f(ws=P[10] + 8) == c["GDR_ERR_ALIGN"]
    assert f(nbytes=need - 1) == c["GDR_ERR_WORKSPACE"]
    assert f(ws=P[2] + 1024) == c["GDR_ERR_ALIAS"]          # workspace inside v
    assert f(chunk=24) == c["GDR_ERR_UNSUPPORTED"]
    assert f(ptrs=[None] + P[1:7]) == c["GDR_ERR_NULL"]
    # the fused kernel's fp32 chunk limit does not apply here: validation passes
    # up to the launch, which is not reached because the pointers are checked first
    assert f(ws=P[0]) == c["GDR_ERR_ALIAS"]


def test_chunk_phase_validation(lib):
    c = _codes()
    need = _ws_size(lib)[1]

    def intra(ptrs=None, ws=P[10], nbytes=None, T=64, chunk=16):
        p = list(P[:6]) if ptrs is None else ptrs
        return lib.gdr_chunk_intra(*p, 1, 2, T, 16, 16, chunk, 1, ws, need if nbytes is None else nbytes, None)

    def scan(ws=P[10], nbytes=None, S0=None, o=P[6], S_out=None, chunk=16):
        return lib.gdr_chunk_scan(ws, need if nbytes is None else nbytes, S0, o, S_out,
                                  1, 2, 64, 16, 16, chunk, 1, None)

    assert intra(ptrs=[None] + P[1:6]) == c["GDR_ERR_NULL"]
    assert intra(ws=None) == c["GDR_ERR_NULL"]
    assert intra(T=0) == c["GDR_ERR_SHAPE"]
    assert intra(chunk=8) == c["GDR_ERR_UNSUPPORTED"]
    assert intra(nbytes=need - 16) == c["GDR_ERR_WORKSPACE"]
    assert intra(ws=P[3] + 64) == c["GDR_ERR_ALIAS"]          # workspace inside alpha
    assert intra(ptrs=P[:5] + [P[5] + 4]) == c["GDR_ERR_ALIGN"]
    assert scan(ws=None) == c["GDR_ERR_NULL"]
    assert scan(o=None) == c["GDR_ERR_NULL"]
    assert scan(nbytes=need - 1) == c["GDR_ERR_WORKSPACE"]
    assert scan(o=P[10] + 256) == c["GDR_ERR_ALIAS"]          # o inside the workspace
    assert scan(S0=P[8], S_out=P[8] + 64) == c["GDR_ERR_ALIAS"]
    assert scan(S_out=P[8] + 8) == c["GDR_ERR_ALIGN"]
    assert scan(chunk=128) == c["GDR_ERR_UNSUPPORTED"]


def test_decode_validation(lib):
    c = _codes()
    f = lambda ptrs, N=4, H=2, dk=16, dv=16, dtype=1: lib.gdr_decode_step(*ptrs, N, H, dk, dv, dtype, None)
    assert f([None] + P[1:8]) == c["GDR_ERR_NULL"]
    assert f(P[:8], N=0) == c["GDR_ERR_SHAPE"]
    assert f(P[:8], dtype=-1) == c["GDR_ERR_DTYPE"]
    assert f(P[:8], dk=24) == c["GDR_ERR_UNSUPPORTED"]
    assert f(P[:6] + [P[6] + 2, P[7]]) == c["GDR_ERR_ALIGN"]
    assert f(P[:6] + [P[6], P[6] + 512]) == c["GDR_ERR_ALIAS"]     # o inside S


def test_mlstm_validation(lib):
    c = _codes()

    def f(q=P[0], k=P[1], v=P[2], it=P[3], ft=P[4], C0=None, n0=None, m0=None, h=P[5],
          Co=None, no=None, mo=None, B=1, H=2, T=64, dk=16, dv=16, chunk=64, dtype=1):
        return lib.gdr_mlstm_fwd(q, k, v, it, ft, C0, n0, m0, h, Co, no, mo, B, H, T, dk, dv, chunk, dtype, None)

    assert f(q=None) == c["GDR_ERR_NULL"]
    assert f(C0=P[6]) == c["GDR_ERR_NULL"]                 # partial initial state
    assert f(Co=P[6], no=P[7]) == c["GDR_ERR_NULL"]        # partial final state
    assert f(T=-3) == c["GDR_ERR_SHAPE"]
    assert f(dtype=2) == c["GDR_ERR_DTYPE"]
    assert f(dk=512) == c["GDR_ERR_UNSUPPORTED"]
    assert f(dk=256, dtype=0) == c["GDR_ERR_UNSUPPORTED"]
    assert f(chunk=8) == c["GDR_ERR_UNSUPPORTED"]
    assert f(it=P[3] + 4) == c["GDR_ERR_ALIGN"]
    assert f(h=P[0]) == c["GDR_ERR_ALIAS"]
    # n_out may not be n0 (all value tiles of a head read n0)
    assert f(C0=P[6], n0=P[7], m0=P[8], Co=P[9], no=P[7], mo=P[10]) == c["GDR_ERR_ALIAS"]


def test_mlstm_ws_validation(lib):
    c = _codes()
    n = ctypes.c_size_t(0)
    assert lib.gdr_mlstm_workspace_size(1, 2, 64, 16, 16, 64, 1, ctypes.byref(n)) == c["GDR_OK"]
    # record: H and V^T (C*dv each) + K~^T (dk*C) in the input dtype, then N, F, A (fp32)
    assert n.value == 2 * 1 * ((16 * 64 * 2 + 16 * 64) * 2 + 3 * 64 * 4)
    need = n.value

    def f(ws=P[12], nbytes=need, dtype=1, dk=16, dv=16, h=P[5]):
        return lib.gdr_mlstm_fwd_ws(P[0], P[1], P[2], P[3], P[4], None, None, None, h, None, None, None,
                                    1, 2, 64, dk, dv, 64, dtype, ws, nbytes, None)

    assert f(ws=None) == c["GDR_ERR_NULL"]
    assert f(ws=P[12] + 4) == c["GDR_ERR_ALIGN"]
    assert f(nbytes=need - 16) == c["GDR_ERR_WORKSPACE"]
    assert f(ws=P[2] + 512) == c["GDR_ERR_ALIAS"]
    assert f(h=P[0]) == c["GDR_ERR_ALIAS"]
    assert f(dtype=0, dv=256) == c["GDR_ERR_UNSUPPORTED"]      # fp32 d_v > 128 on this path


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import matrix_memory_rnn_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "lib_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        m.load_library()


def test_noalloc_rejects_a_head_larger_than_its_scratch(lib):
    """gdr_chunk_fwd_noalloc checks the per-head record size against its static
    scratch array on the host, before touching the GPU."""
    c = _codes()
    assert c["GDR_ERR_TOO_LARGE"] == -9
    p = P[:7]
    # one head of 100,000 tokens at d = 128, C = 64, bf16 needs 1563 records of
    # 74,240 B (116 MB), more than the 64 MiB array
    st = lib.gdr_chunk_fwd_noalloc(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], None,
                                   1, 2, 100000, 128, 128, 64, 1, None)
    assert st == c["GDR_ERR_TOO_LARGE"]
    assert "scratch" in lib.gdr_status_string(st).decode()
    # argument errors come first, as for the other entry points
    st = lib.gdr_chunk_fwd_noalloc(None, p[1], p[2], p[3], p[4], p[5], None, p[6], None,
                                   1, 2, 64, 16, 16, 16, 1, None)
    assert st == c["GDR_ERR_NULL"]
