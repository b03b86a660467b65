"""The C ABI without a GPU: the library loads, exports every symbol that
include/nrc.h declares, and rejects bad arguments on the host before any
launch (so these calls never touch a device)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nrc.h")

EINVAL, ENOTSUP = -22, -95


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|int64_t|const char\*|void)\s+(nrc_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import norm_rope_cache_amd as m

    if not os.path.exists(m.library_path()):
        from norm_rope_cache_amd import build

        build.build()
    return m._load()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("nrc_context_norms", "nrc_context_kv_project", "nrc_context_kv_store", "nrc_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s


def test_abi_version(lib):
    assert lib.nrc_abi_version() == 1


def _err(lib):
    return lib.nrc_last_error().decode()


FAKE = ctypes.c_void_p(0x10000)  # an aligned non-NULL address that is never dereferenced
MISALIGNED = ctypes.c_void_p(0x10002)


def test_norms_argument_checks(lib):
    f = lib.nrc_context_norms
    assert f(FAKE, 4, 4096, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == ENOTSUP
    assert "8192" in _err(lib)
    assert f(FAKE, -1, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == EINVAL
    assert f(FAKE, 4, 8192, None, None, 0, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == EINVAL
    assert f(None, 4, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == EINVAL
    assert f(MISALIGNED, 4, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == EINVAL
    assert f(FAKE, 4, 8192, MISALIGNED, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None) == EINVAL
    # T == 0 is a no-op that touches nothing
    assert f(None, 0, 8192, None, None, 3, 1e-6, 1e-6, 0.0, 0.0, None, None) == 0


def test_norms_ex_argument_checks(lib):
    f = lib.nrc_context_norms_ex
    ok = dict(x=FAKE, T=4, D=8192, hw=None, hk=0, pw=None, pk=0, L=1, flags=0, out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["T"], a["D"], a["hw"], a["hk"], a["pw"], a["pk"], a["L"], 1e-6, 1e-6, 0.0, 0.0,
                 a["flags"], a["out"], None)

    assert call(D=4096) == ENOTSUP
    assert call(T=-1) == EINVAL
    assert call(L=0) == EINVAL
    assert call(hk=3, hw=FAKE) == EINVAL
    assert call(pk=-1) == EINVAL
    assert call(hk=1) == EINVAL            # bf16 kind without a pointer
    assert call(hw=FAKE) == EINVAL         # pointer with kind none
    assert call(pk=2) == EINVAL
    assert call(flags=4) == EINVAL
    assert call(x=None) == EINVAL
    assert call(out=MISALIGNED) == EINVAL
    assert call(hk=2, hw=MISALIGNED) == EINVAL
    assert call(T=0, x=None, out=None) == 0


def test_store_ex_argument_checks(lib):
    f = lib.nrc_context_kv_store_ex
    P = ctypes.c_void_p
    slots = (P * 2)(FAKE.value, None)
    caches = (P * 2)(FAKE.value, None)
    rows = (ctypes.c_int64 * 2)(8, 0)

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, kls=1024 * 16, krs=1024, vls=1024 * 16, vrs=1024, pos=FAKE, slots=slots,
                 rows=rows, T=16, cs=None, maxp=0, caches=caches, nb=64, bs=16, bstr=8 * 16 * 128, pstr=128,
                 hstr=16 * 128, H=8, L=2)
        a.update(kw)
        return f(a["k"], a["v"], a["kls"], a["krs"], a["vls"], a["vrs"], a["pos"], a["slots"], a["rows"], a["T"],
                 a["cs"], a["maxp"], a["caches"], a["nb"], a["bs"], a["bstr"], a["pstr"], a["hstr"], a["H"], a["L"],
                 1e-6, None)

    assert call(rows=None) == EINVAL
    assert call(rows=(ctypes.c_int64 * 2)(17, 0)) == EINVAL     # rows > T
    assert call(rows=(ctypes.c_int64 * 2)(-1, 0)) == EINVAL
    assert call(pstr=-128) == EINVAL
    assert call(hstr=16 * 128 + 4) == ENOTSUP                  # not a multiple of 8 elements
    assert call(H=6) == ENOTSUP
    assert call(caches=(P * 2)(None, None)) == EINVAL          # a storing layer without a cache
    assert call(caches=(P * 2)(MISALIGNED.value, None)) == EINVAL
    assert call(k=MISALIGNED) == EINVAL
    # nothing to store: every layer without slots, or zero rows
    assert call(slots=(P * 2)(None, None), k=None, v=None) == 0
    assert call(rows=(ctypes.c_int64 * 2)(0, 5), k=None, v=None) == 0


def test_boundary_argument_checks(lib):
    f = lib.nrc_draft_boundary
    ok = dict(br=FAKE, m=4, D=8192, s=FAKE, sk=0, a=FAKE, b=FAKE, pw=None, pk=0, qw=None, qk=0, flags=0, so=None,
              out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["br"], a["m"], a["D"], a["s"], a["sk"], a["a"], a["b"], a["pw"], a["pk"], a["qw"], a["qk"],
                 1e-6, 1e-6, 0.0, 0.0, a["flags"], a["so"], a["out"], None)

    assert call(D=4096) == ENOTSUP
    assert call(m=-1) == EINVAL
    assert call(sk=2) == EINVAL
    assert call(pk=4, pw=FAKE) == EINVAL
    assert call(pk=3) == EINVAL            # FP16 kind without a pointer
    assert call(qw=FAKE) == EINVAL         # pointer with kind none
    assert call(flags=4) == EINVAL
    assert call(a=None) == EINVAL
    assert call(so=MISALIGNED) == EINVAL
    assert call(s=MISALIGNED) == EINVAL
    assert call(m=0, br=None, s=None, a=None, b=None, out=None) == 0


def test_project_argument_checks(lib):
    f = lib.nrc_context_kv_project
    assert f(FAKE, FAKE, FAKE, 0, 8, 8192, 1024, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, 1, -1, 8192, 1024, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, 1, 8, 8100, 1024, None) == ENOTSUP
    assert f(FAKE, FAKE, FAKE, 1, 8, 8192, 1000, None) == ENOTSUP
    assert f(FAKE, None, FAKE, 1, 8, 8192, 1024, None) == EINVAL
    assert f(FAKE, FAKE, MISALIGNED, 1, 8, 8192, 1024, None) == EINVAL
    assert f(None, None, None, 2, 0, 8192, 1024, None) == 0


def test_project_split_workspace_and_argument_checks(lib):
    """The split form's workspace query (no GPU here: the library assumes 256
    CUs, as on MI355X) and its argument checks, all before any launch."""
    q = lib.nrc_context_kv_project_workspace_bytes
    q.restype = ctypes.c_int64
    # long workload: 256 x 256 tiles fill the CUs, no split
    assert q(4, 16384, 8192, 1024) == 0
    # a 512-row prefill: 32 tiles of 256 x 256, eight slices
    assert q(4, 512, 8192, 1024) == 8 * 4 * 512 * 1024 * 4
    # 256 rows: 16 tiles of 256 x 256, still eight slices (the cap for that tile)
    assert q(4, 256, 8192, 1024) == 8 * 4 * 256 * 1024 * 4
    # 2000 rows: 128 tiles of 256 x 256, two slices
    assert q(4, 2000, 8192, 1024) == 2 * 4 * 2000 * 1024 * 4
    # N = 384: 128 x 128 tiles (18 of them), sixteen slices
    assert q(2, 300, 8192, 384) == 16 * 2 * 300 * 384 * 4
    # 16 rows: sixteen slices at most
    assert q(2, 16, 8192, 256) == 16 * 2 * 16 * 256 * 4
    # D = 1024 (32 stages): slices of at least 4 stages, an even number each
    assert q(2, 16, 1024, 256) == 8 * 2 * 16 * 256 * 4
    # D = 2048 (64 stages): sixteen slices of 4 stages
    assert q(2, 16, 2048, 256) == 16 * 2 * 16 * 256 * 4
    assert q(4, 0, 8192, 1024) == 0
    assert q(0, 512, 8192, 1024) == EINVAL
    assert q(4, 512, 8100, 1024) == ENOTSUP
    assert q(4, 512, 8192, 1000) == ENOTSUP
    f = lib.nrc_context_kv_project_split
    need = 8 * 4 * 512 * 1024 * 4
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, None, need, None) == EINVAL
    assert "workspace" in _err(lib)
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, FAKE, need - 1, None) == EINVAL
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, MISALIGNED, need, None) == EINVAL
    assert f(FAKE, FAKE, 2, FAKE, 4, 512, 8192, 1024, FAKE, need, None) == EINVAL
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1000, FAKE, need, None) == ENOTSUP
    assert f(None, None, 0, None, 4, 0, 8192, 1024, None, 0, None) == 0


def test_project_timed_argument_checks(lib):
    """The clock-stamped projection rejects bad host outputs, stamps and shapes
    before touching a device (no GPU here: the library assumes 256 CUs, so
    8 * 256 stamps are required)."""
    f = lib.nrc_context_kv_project_timed
    wg, khz = ctypes.c_int32(7), ctypes.c_int32(0)
    n = 8 * 256
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, FAKE, n, None, ctypes.byref(khz), None) == EINVAL
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, FAKE, n, ctypes.byref(wg), None, None) == EINVAL
    assert f(FAKE, FAKE, 2, FAKE, 4, 512, 8192, 1024, FAKE, n, ctypes.byref(wg), ctypes.byref(khz), None) == EINVAL
    assert wg.value == 0, "workgroups is cleared on every call"
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1000, FAKE, n, ctypes.byref(wg), ctypes.byref(khz), None) == ENOTSUP
    assert f(FAKE, FAKE, 0, FAKE, 0, 512, 8192, 1024, FAKE, n, ctypes.byref(wg), ctypes.byref(khz), None) == EINVAL
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, None, n, ctypes.byref(wg), ctypes.byref(khz), None) == EINVAL
    assert "stamps" in _err(lib)
    odd = ctypes.c_void_p(0x10004)  # 4- but not 8-byte aligned
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, odd, n, ctypes.byref(wg), ctypes.byref(khz), None) == EINVAL
    assert f(FAKE, FAKE, 0, FAKE, 4, 512, 8192, 1024, FAKE, n - 1, ctypes.byref(wg), ctypes.byref(khz), None) == EINVAL
    assert str(n) in _err(lib)

def _store(lib, **kw):
    a = dict(k=FAKE, v=FAKE, kls=1024 * 16, krs=1024, vls=1024 * 16, vrs=1024, pos=FAKE, slots=None, rows=16,
             T=16, cs=FAKE, maxp=4096, caches=None, nb=64, bs=16, H=8, L=2, eps=1e-6)
    a.update(kw)
    L = a["L"]
    arr = ctypes.c_void_p * max(L, 1)
    slots = a["slots"] if a["slots"] is not None else arr(*([0x20000] * max(L, 1)))
    caches = a["caches"] if a["caches"] is not None else arr(*([0x30000] * max(L, 1)))
    return lib.nrc_context_kv_store(a["k"], a["v"], a["kls"], a["krs"], a["vls"], a["vrs"], a["pos"], slots,
                                    a["rows"], a["T"], a["cs"], a["maxp"], caches, a["nb"], a["bs"], a["H"], L,
                                    a["eps"], None)


def test_store_argument_checks(lib):
    assert _store(lib, L=0) == EINVAL
    assert _store(lib, H=0) == EINVAL
    assert _store(lib, H=6) == ENOTSUP
    assert "power of two" in _err(lib)
    assert _store(lib, rows=17) == EINVAL
    assert _store(lib, rows=-1) == EINVAL
    assert _store(lib, nb=1 << 27, bs=16) == ENOTSUP  # 2^31 slots
    assert _store(lib, nb=0) == EINVAL
    assert _store(lib, k=None) == EINVAL
    assert _store(lib, v=MISALIGNED) == EINVAL
    assert _store(lib, krs=1020) == EINVAL  # not a multiple of 8 elements
    assert _store(lib, pos=None) == EINVAL  # RoPE without positions
    assert _store(lib, maxp=0) == EINVAL
    arr = ctypes.c_void_p * 2
    assert _store(lib, slots=arr(0x20000, 0)) == EINVAL  # NULL slots of layer 1
    assert _store(lib, caches=arr(0x30000, 0x30008)) == EINVAL  # misaligned cache of layer 1
    # rows == 0 (and T == 0) are no-ops that touch nothing
    assert _store(lib, rows=0, k=None, v=None, slots=None) == 0
    assert _store(lib, rows=0, T=0) == 0


def test_project_store_argument_checks(lib):
    """The one-call projection + store checks the operands of both parts
    before it launches anything (every call here fails, or does nothing, on
    the host; the library assumes 256 CUs, so the 512-row shape splits)."""
    f = lib.nrc_context_kv_project_store
    need = 8 * 4 * 512 * 1024 * 4
    arr = ctypes.c_void_p * 4
    slots, caches = arr(*([0x20000] * 4)), arr(*([0x30000] * 4))

    def call(**kw):
        a = dict(normed=FAKE, w=FAKE, layout=0, kv=FAKE, L=4, T=512, D=8192, N=1024, ws=FAKE, wsb=need, pos=FAKE,
                 slots=slots, rows=512, cs=FAKE, maxp=4096, caches=caches, nb=64, bs=16, eps=1e-6)
        a.update(kw)
        return f(a["normed"], a["w"], a["layout"], a["kv"], a["L"], a["T"], a["D"], a["N"], a["ws"], a["wsb"],
                 a["pos"], a["slots"], a["rows"], a["cs"], a["maxp"], a["caches"], a["nb"], a["bs"], a["eps"], None)

    assert call(layout=2) == EINVAL
    assert call(N=1000) == ENOTSUP
    assert call(rows=513) == EINVAL
    assert call(rows=-1) == EINVAL
    assert call(kv=MISALIGNED) == EINVAL
    assert call(ws=None) == EINVAL
    assert "workspace" in _err(lib)
    assert call(wsb=need - 1) == EINVAL
    assert call(slots=None) == EINVAL
    assert call(slots=arr(0x20000, 0x20000, 0, 0x20000)) == EINVAL
    assert "layer 2" in _err(lib)
    assert call(caches=arr(0x30000, 0x30008, 0x30000, 0x30000)) == EINVAL  # misaligned cache of layer 1
    assert call(pos=None) == EINVAL  # RoPE without positions
    assert call(nb=0) == EINVAL
    # N = 384: three KV heads, not a power of two (the projection alone would accept it)
    need3 = lib.nrc_context_kv_project_workspace_bytes(4, 512, 8192, 384)
    assert call(N=384, wsb=need3) == ENOTSUP
    assert "power of two" in _err(lib)
    assert call(normed=None, w=None, kv=None, T=0, rows=0, ws=None, wsb=0) == 0


def test_fused_argument_checks(lib):
    f = lib.nrc_context_hidden_norm
    assert f(FAKE, 4, 4096, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, FAKE, None) == ENOTSUP
    assert f(FAKE, 4, 8192, None, None, 0, 1e-6, 1e-6, 0.0, 0.0, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, FAKE, None, None) == EINVAL
    assert f(FAKE, 4, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, MISALIGNED, FAKE, None) == EINVAL
    assert f(None, 0, 8192, None, None, 1, 1e-6, 1e-6, 0.0, 0.0, None, None, None) == 0
    g = lib.nrc_context_kv_project_fused
    assert g(FAKE, FAKE, None, 0.0, FAKE, FAKE, 0, 8, 8192, 1024, None) == EINVAL
    assert g(FAKE, FAKE, None, 0.0, FAKE, FAKE, 1, 8, 4096, 1024, None) == ENOTSUP
    assert g(FAKE, FAKE, None, 0.0, FAKE, FAKE, 1, 8, 8192, 1000, None) == ENOTSUP
    assert g(FAKE, None, None, 0.0, FAKE, FAKE, 1, 8, 8192, 1024, None) == EINVAL
    assert g(FAKE, FAKE, MISALIGNED, 0.0, FAKE, FAKE, 1, 8, 8192, 1024, None) == EINVAL
    assert g(None, None, None, 0.0, None, None, 2, 0, 8192, 1024, None) == 0


def test_check_scalars_argument_checks(lib):
    assert lib.nrc_check_scalars(FAKE, None, None, 4, None) == EINVAL
    assert lib.nrc_check_scalars(FAKE, FAKE, None, -1, None) == EINVAL
    assert lib.nrc_check_scalars(None, None, None, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No fallback path: with libnrc.so missing, every call raises."""
    import norm_rope_cache_amd as m

    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        m.abi_version()
