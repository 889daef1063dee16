"""C-ABI checks that need no GPU: the library loads, exports every function that
include/gdr.h declares, and rejects bad arguments with the documented codes
before enqueuing anything (all pointers here are fake and never dereferenced).

The same module also runs against libgdr_hostsan.so, whose entry points' host
code carries AddressSanitizer and UndefinedBehaviorSanitizer checks: the last
test starts a second pytest process on this file with that library selected
(GDR_ABI_LIB) and the sanitizer runtime preloaded, so every validation path
below also runs under the sanitizers."""
import ctypes
import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")
PKG = os.path.join(ROOT, "matrix_memory_rnn_amd")
LIB = os.environ.get("GDR_ABI_LIB") or os.path.join(PKG, "libgdr.so")
LIB_DEBUG = os.path.join(PKG, "libgdr_debug.so")
LIB_HOSTSAN = os.path.join(PKG, "libgdr_hostsan.so")

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
    if os.environ.get("GDR_ABI_LIB"):
        return m.declare(ctypes.CDLL(LIB))   # no torch under the sanitizer runtime
    return m.load_library()


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("gdr_chunk_fwd", "gdr_chunk_fwd_ws", "gdr_chunk_workspace_size", "gdr_chunk_intra",
              "gdr_chunk_scan", "gdr_decode_step", "gdr_mlstm_fwd", "gdr_mlstm_fwd_ws",
              "gdr_mlstm_workspace_size", "gdr_status_string", "gdr_version"):
        assert n in names


@pytest.mark.parametrize("path", [LIB, LIB_DEBUG, LIB_HOSTSAN])
def test_library_exports_every_declared_symbol(path):
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not built")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdr_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_symbols_resolve_through_dlopen(lib):
    for n in _declared():
        assert hasattr(lib, n)
    assert lib.gdr_version() == 200
    assert lib.gdr_debug_violation().decode() == ""


def test_debug_library_says_so():
    """libgdr_debug.so reports itself as the checking build; libgdr.so does not."""
    if not os.path.exists(LIB_DEBUG) or os.environ.get("GDR_ABI_LIB"):
        pytest.skip("libgdr_debug.so not built")
    import matrix_memory_rnn_amd as m
    dbg = m.declare(ctypes.CDLL(LIB_DEBUG))
    rel = m.declare(ctypes.CDLL(os.path.join(PKG, "libgdr.so")))
    assert dbg.gdr_debug_build() == 1 and rel.gdr_debug_build() == 0
    assert _codes()["GDR_ERR_PRECONDITION"] == -10
    assert "gdr_debug_violation" in dbg.gdr_status_string(-10).decode()
    # host validation runs first in the debug build too: nothing reaches the GPU
    p = P[:7]
    assert dbg.gdr_chunk_fwd(None, *p[1:6], None, p[6], None, 1, 2, 64, 16, 16, 16, 1, None) == -1


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


def test_muir_validation(lib):
    c = _codes()
    need = _ws_size(lib)[1]

    def f(zq=None, a_log=P[11], gamma=None, ws=P[10], nbytes=None, o=P[6], ptrs=None):
        p = list(P[:6]) if ptrs is None else ptrs
        return lib.gdr_muir_chunk_fwd_ws(*p, zq, a_log, gamma, None, o, None, 1, 2, 64, 16, 16, 16, 1,
                                         ws, need if nbytes is None else nbytes, None)

    def g(zq=None, a_log=P[11], gamma=None, S=P[7], o=P[6], N=4, dk=16):
        return lib.gdr_muir_decode_step(*P[:6], zq, a_log, gamma, S, o, N, 2, dk, 16, 1, None)

    assert f(a_log=None) == c["GDR_ERR_NULL"]
    assert f(ptrs=[None] + P[1:6]) == c["GDR_ERR_NULL"]
    assert f(zq=P[12] + 8) == c["GDR_ERR_ALIGN"]
    assert f(a_log=P[11] + 2) == c["GDR_ERR_ALIGN"]          # float32 arrays: 4-byte alignment
    assert f(gamma=P[12] + 1) == c["GDR_ERR_ALIGN"]
    assert f(o=P[11]) == c["GDR_ERR_ALIAS"]                  # o over a_log
    assert f(nbytes=need - 1) == c["GDR_ERR_WORKSPACE"]
    assert f(ws=P[12], zq=P[12] + 256) == c["GDR_ERR_ALIAS"]  # z_q inside the workspace
    assert g(a_log=None) == c["GDR_ERR_NULL"]
    assert g(S=None) == c["GDR_ERR_NULL"]
    assert g(N=0) == c["GDR_ERR_SHAPE"]
    assert g(dk=24) == c["GDR_ERR_UNSUPPORTED"]
    assert g(gamma=P[12] + 2) == c["GDR_ERR_ALIGN"]
    assert g(o=P[11]) == c["GDR_ERR_ALIAS"]


def test_bwd_validation(lib):
    c = _codes()

    def need(T=64, chunk=16, dtype=1):
        n = ctypes.c_size_t(7)
        st = lib.gdr_chunk_bwd_workspace_size(1, 2, T, 16, 16, chunk, dtype, ctypes.byref(n))
        return st, n.value

    def f(ptrs=None, dO=P[7], dS_T=None, outs=None, ws=P[14], nbytes=None, chunk=16, T=64):
        p = list(P[:6]) if ptrs is None else ptrs
        o = [P[8], P[9], P[10], P[11], P[12], P[13], None] if outs is None else outs
        n = need(64, 16)[1] if nbytes is None else nbytes
        return lib.gdr_chunk_bwd(*p, None, dO, dS_T, *o, 1, 2, T, 16, 16, chunk, 1, ws, n, 0, None)

    st, n = need()
    assert st == c["GDR_OK"] and n > 0
    assert need(T=0) == (c["GDR_ERR_SHAPE"], 0)
    assert need(chunk=128)[0] == c["GDR_ERR_UNSUPPORTED"]
    assert lib.gdr_chunk_bwd_workspace_size(1, 2, 64, 16, 16, 16, 1, None) == c["GDR_ERR_NULL"]
    assert f(dO=None) == c["GDR_ERR_NULL"]
    assert f(ws=None) == c["GDR_ERR_NULL"]
    assert f(outs=[None, P[9], P[10], P[11], P[12], P[13], None]) == c["GDR_ERR_NULL"]
    assert f(T=0) == c["GDR_ERR_SHAPE"]
    assert f(chunk=8) == c["GDR_ERR_UNSUPPORTED"]
    assert f(dS_T=P[15] + 8) == c["GDR_ERR_ALIGN"]
    assert f(nbytes=n - 1) == c["GDR_ERR_WORKSPACE"]
    assert f(outs=[P[0], P[9], P[10], P[11], P[12], P[13], None]) == c["GDR_ERR_ALIAS"]          # dq over q
    assert f(outs=[P[8], P[8] + 64, P[10], P[11], P[12], P[13], None]) == c["GDR_ERR_ALIAS"]     # dk over dq
    assert f(ws=P[7] + 256) == c["GDR_ERR_ALIAS"]                                               # ws inside dO


def test_rwkv7_validation(lib):
    c = _codes()

    def need(T=64, chunk=16):
        n = ctypes.c_size_t(7)
        st = lib.gdr_rwkv7_workspace_size(1, 2, T, 16, 16, chunk, ctypes.byref(n))
        return st, n.value

    def f(cc=P[3], ws=P[10], nbytes=None, chunk=16, o=P[6], S0=None, S_out=None, dk=16, T=64, q=P[0]):
        n = need()[1] if nbytes is None else nbytes
        return lib.gdr_rwkv7_fwd(q, P[1], P[2], cc, P[4], P[5], S0, o, S_out, 1, 2, T, dk, 16, chunk, 1,
                                 ws, n, None)

    def g(S=P[7], o=P[6], N=4, q=P[0]):
        return lib.gdr_rwkv7_decode_step(q, P[1], P[2], P[3], P[4], P[5], S, o, N, 2, 16, 16, 1, None)

    st, n = need()
    assert st == c["GDR_OK"] and n > 0
    assert need(chunk=64)[0] == c["GDR_ERR_UNSUPPORTED"]
    assert need(T=0) == (c["GDR_ERR_SHAPE"], 0)
    assert lib.gdr_rwkv7_workspace_size(1, 2, 64, 16, 16, 16, None) == c["GDR_ERR_NULL"]
    assert f(cc=None) == c["GDR_ERR_NULL"]
    assert f(ws=None) == c["GDR_ERR_NULL"]
    assert f(T=0) == c["GDR_ERR_SHAPE"]
    assert f(chunk=64) == c["GDR_ERR_UNSUPPORTED"]
    assert f(dk=48) == c["GDR_ERR_UNSUPPORTED"]
    assert f(cc=P[3] + 4) == c["GDR_ERR_ALIGN"]
    assert f(nbytes=n - 1) == c["GDR_ERR_WORKSPACE"]
    assert f(o=P[5] + 32) == c["GDR_ERR_ALIAS"]              # o over u
    assert f(ws=P[3]) == c["GDR_ERR_ALIAS"]                  # workspace over c
    assert f(S0=P[8], S_out=P[8] + 64) == c["GDR_ERR_ALIAS"]
    assert g(S=None) == c["GDR_ERR_NULL"]
    assert g(N=0) == c["GDR_ERR_SHAPE"]
    assert g(S=P[0]) == c["GDR_ERR_ALIAS"]                   # state over q
    assert g(q=P[0] + 4) == c["GDR_ERR_ALIGN"]


def _asan_runtime():
    for clang in ("/opt/rocm/lib/llvm/bin/clang", "clang"):
        try:
            out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                 text=True, timeout=30).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            continue
        if out and os.path.isabs(out) and os.path.exists(out):
            return out
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def test_validation_paths_under_host_sanitizers():
    """Every validation test of this module, run again in a fresh process on
    libgdr_hostsan.so with the ASan runtime preloaded: an out-of-bounds access,
    use after free or undefined behaviour (signed overflow, misaligned access,
    bad shift) in the host-side argument checks aborts that process."""
    if os.environ.get("GDR_ABI_LIB"):
        pytest.skip("already the sanitized run")
    rt = _asan_runtime()
    if not os.path.exists(LIB_HOSTSAN) or rt is None:
        pytest.skip("libgdr_hostsan.so or the ASan runtime is missing")
    env = dict(os.environ, GDR_ABI_LIB=LIB_HOSTSAN, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        "-k", "not host_sanitizers and not fails_loudly"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) >= 10, tail
