"""The no-allocation projection (nrc_context_kv_project_noalloc) through the
C ABI: the same bits as nrc_context_kv_project_split with a caller workspace,
on consecutive calls of shrinking size (the device scratch keeps the previous
call's contents), a shape that does not split, and a shape whose split needs
more scratch than the library holds (refused, nothing written)."""

import ctypes

import numpy as np
import pytest

from helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    import norm_rope_cache_amd as m

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    L = m._load()
    L.nrc_context_kv_project_noalloc.restype = ctypes.c_int32
    L.nrc_context_kv_project_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_void_p]
    return L


SCRATCH = 64 << 20


def _operands(L, T, N, seed, nd=False):
    from norm_rope_cache_amd import synth

    A = to_dev(synth.normal_bf16(seed, (L, T, 8192)))
    B = synth.normal_bf16(seed + 1, (L, 8192, N), std=0.02)
    if nd:
        B = np.ascontiguousarray(np.swapaxes(B, 1, 2))
    return A, to_dev(B)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(lib, A, B, layout, L, T, N, out):
    return lib.nrc_context_kv_project_noalloc(A.data_ptr(), B.data_ptr(), layout, out.data_ptr(), L, T, 8192, N,
                                              _stream())


def _with_workspace(lib, A, B, layout, L, T, N):
    need = lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N)
    assert need >= 0
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((L, T, N), dtype=torch.bfloat16, device="cuda")
    rc = lib.nrc_context_kv_project_split(A.data_ptr(), B.data_ptr(), layout, out.data_ptr(), L, T, 8192, N,
                                          ws.data_ptr(), need, _stream())
    assert rc == 0, lib.nrc_last_error()
    torch.cuda.synchronize()
    return need, to_host(out)


@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_matches_workspace_form_on_shrinking_calls(lib, layout):
    # the largest split that fits the scratch exactly, then smaller splits
    shapes = [(4, 512, 1024), (2, 300, 384), (1, 37, 128)]
    needs = []
    for i, (L, T, N) in enumerate(shapes):
        print(f"noalloc layout={layout} L={L} T={T} N={N}", flush=True)
        A, B = _operands(L, T, N, 7100 + 10 * i, nd=layout == 1)
        need, want = _with_workspace(lib, A, B, layout, L, T, N)
        needs.append(need)
        out = torch.empty((L, T, N), dtype=torch.bfloat16, device="cuda")
        rc = _noalloc(lib, A, B, layout, L, T, N, out)
        assert rc == 0, lib.nrc_last_error()
        torch.cuda.synchronize()
        got = to_host(out)
        assert np.array_equal(got, want), f"noalloc vs workspace form, shape {(L, T, N)}"
    assert needs[0] == SCRATCH and 0 < needs[2] < needs[1] < needs[0], needs


def test_noalloc_unsplit_shape_is_the_one_pass_projection(lib):
    L, T, N = 4, 4096, 1024
    A, B = _operands(L, T, N, 7200)
    assert lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N) == 0
    want = torch.empty((L, T, N), dtype=torch.bfloat16, device="cuda")
    assert lib.nrc_context_kv_project(A.data_ptr(), B.data_ptr(), want.data_ptr(), L, T, 8192, N, _stream()) == 0
    got = torch.empty_like(want)
    assert _noalloc(lib, A, B, 0, L, T, N, got) == 0, lib.nrc_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(to_host(got), to_host(want))


def test_noalloc_refuses_a_split_beyond_the_scratch(lib):
    L, T, N = 4, 700, 1024  # eight 256 x 256 slices of 700 rows: 91.75 MB of partial sums
    assert lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N) > SCRATCH
    A, B = _operands(L, T, N, 7300)
    out = torch.zeros((L, T, N), dtype=torch.bfloat16, device="cuda")
    rc = _noalloc(lib, A, B, 0, L, T, N, out)
    assert rc == -22
    assert b"scratch" in lib.nrc_last_error()
    torch.cuda.synchronize()
    assert not bool(out.view(torch.int16).any())
