"""ctypes view of the CPU oracle (oracle/oracle.c) over numpy arrays.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's cpu_baseline leg. The product package never imports it, and it
imports nothing from the product package. bf16 tensors are numpy uint16
arrays holding the bf16 bit patterns.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("NRC_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

D = 8192
HEAD_DIM = 64

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.nrc_oracle_bf16.argtypes = [_f32]
        L.nrc_oracle_bf16.restype = ctypes.c_uint16
        L.nrc_oracle_rs.argtypes = [_f32]
        L.nrc_oracle_rs.restype = _f32
        L.nrc_oracle_bf16_array.argtypes = [_f32p, _u16p, _i64]
        L.nrc_oracle_bf16_array.restype = None
        L.nrc_oracle_rs_array.argtypes = [_f32p, _f32p, _i64]
        L.nrc_oracle_rs_array.restype = None
        L.nrc_oracle_sumsq_row.argtypes = [_f32p]
        L.nrc_oracle_sumsq_row.restype = _f32
        L.nrc_oracle_sumsq_head.argtypes = [_f32p]
        L.nrc_oracle_sumsq_head.restype = _f32
        L.nrc_oracle_context_norms.argtypes = [_u16p, _i64, _i64, _u16p, _u16p, _i32, _f32, _f32, _f32, _f32, _u16p]
        L.nrc_oracle_context_norms.restype = _i32
        L.nrc_oracle_context_norms_ex.restype = _i32
        L.nrc_oracle_context_norms_ex.argtypes = [_u16p, _i64, _i64, ctypes.c_void_p, _i32, ctypes.c_void_p, _i32, _i32,
                                                  _f32, _f32, _f32, _f32, _i32, _u16p]
        L.nrc_oracle_context_kv_store_ex.restype = _i32
        L.nrc_oracle_context_kv_store_ex.argtypes = [
            _u16p, _i32, _i64, _i32, _i64p, ctypes.POINTER(ctypes.c_void_p), _i64p, _u16p, _i64,
            ctypes.POINTER(ctypes.c_void_p), _i64p, _i64, _i64, _i64, _i64, _i64, _f32]
        L.nrc_oracle_kv_project_nd.restype = _i32
        L.nrc_oracle_kv_project_nd.argtypes = [_u16p, _u16p, _f32p, _i32, _i64, _i64, _i64]
        L.nrc_oracle_f16_to_f32.restype = _f32
        L.nrc_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.nrc_oracle_draft_boundary.restype = _i32
        L.nrc_oracle_draft_boundary.argtypes = [
            _u16p, _i64, ctypes.c_void_p, _i32, _f32p, _f32p, ctypes.c_void_p, _i32, ctypes.c_void_p, _i32,
            _f32, _f32, _f32, _f32, _i32, _f32p, _u16p]
        L.nrc_oracle_hidden_norm.argtypes = [_u16p, _i64, _i64, _u16p, _f32, _f32, _f32, _u16p, _f32p]
        L.nrc_oracle_hidden_norm.restype = _i32
        L.nrc_oracle_kv_project.argtypes = [_u16p, _u16p, _f32p, _i32, _i64, _i64, _i64]
        L.nrc_oracle_kv_project.restype = _i32
        L.nrc_oracle_knorm_rope_head.argtypes = [_u16p, _u16p, _f32, _u16p]
        L.nrc_oracle_knorm_rope_head.restype = None
        L.nrc_oracle_cache_offset.argtypes = [_i64, _i64, _i32, _i32]
        L.nrc_oracle_cache_offset.restype = _i64
        L.nrc_oracle_context_kv_store.argtypes = [
            _u16p, _i32, _i64, _i32, _i64p, _i64p, _i64, _u16p, _i64, _u16p, _i64, _i64, _f32]
        L.nrc_oracle_context_kv_store.restype = _i32
        L.nrc_oracle_chain.argtypes = [
            _u16p, _i64, _u16p, _u16p, _i32, _f32, _f32, _u16p, _i32, _i64p, _i64p, _i64, _u16p, _i64,
            _u16p, _i64, _i64, _f32, _u16p, _u16p]
        L.nrc_oracle_chain.restype = _i32
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


class OracleError(RuntimeError):
    pass


def _check(st, what):
    if st != 0:
        raise OracleError(f"{what}: oracle precondition failed ({st})")


# ------------------------------------------------------------------ scalars

def bf16(x):
    """f32 -> bf16 bits (round to nearest even; NaN -> 0x7FC0), elementwise."""
    shape = np.shape(x)
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().nrc_oracle_bf16_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out.reshape(shape)


def rs(v):
    """1 / sqrt(v), both correctly rounded in FP32, elementwise."""
    shape = np.shape(v)
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    out = np.empty(v.shape, dtype=np.float32)
    lib().nrc_oracle_rs_array(_ptr(v, ctypes.c_float), _ptr(out, ctypes.c_float), v.size)
    return out.reshape(shape)


def sumsq_row(u):
    u = _c(np.asarray(u, dtype=np.float32), np.float32)
    assert u.shape == (D,)
    return np.float32(lib().nrc_oracle_sumsq_row(_ptr(u, ctypes.c_float)))


def sumsq_head(k):
    k = _c(np.asarray(k, dtype=np.float32), np.float32)
    assert k.shape == (HEAD_DIM,)
    return np.float32(lib().nrc_oracle_sumsq_head(_ptr(k, ctypes.c_float)))


# ------------------------------------------------------------------- chain

def context_norms(x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, hidden_center=0.0, pre_center=0.0):
    """x [T, 8192] bf16 bits -> [L, T, 8192] bf16 bits."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    assert x.shape == (T, D)
    hw = None if hidden_w is None else _c(hidden_w, np.uint16)
    pw = None if pre_w is None else _c(pre_w, np.uint16)
    if hw is not None:
        assert hw.shape == (D,)
    if pw is not None:
        assert pw.shape == (L, D)
    out = np.empty((L, T, D), dtype=np.uint16)
    st = lib().nrc_oracle_context_norms(
        _ptr(x, ctypes.c_uint16), T, D, _ptr(hw, ctypes.c_uint16), _ptr(pw, ctypes.c_uint16), L,
        hidden_eps, pre_eps, hidden_center, pre_center, _ptr(out, ctypes.c_uint16))
    _check(st, "context_norms")
    return out


def _weight(w, shape):
    """(kind, contiguous array) of a norm weight: None, bf16 bits (uint16) or
    FP32 values (float32)."""
    if w is None:
        return 0, None
    w = np.asarray(w)
    if w.dtype == np.uint16:
        kind = 1
    elif w.dtype == np.float32:
        kind = 2
    else:
        raise TypeError(f"norm weight of dtype {w.dtype}: expected uint16 (bf16 bits) or float32")
    w = np.ascontiguousarray(w)
    assert w.shape == shape, (w.shape, shape)
    return kind, w


def context_norms_ex(x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, hidden_center=0.0, pre_center=0.0,
                     hidden_input_scale=False, pre_input_scale=False):
    """The norms with bf16 or FP32 weights (uint16 bits or float32 arrays,
    None for weightless) and, per norm, the weight scaling the input instead
    of the output. x [T, 8192] bf16 bits -> [L, T, 8192] bf16 bits."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    assert x.shape == (T, D)
    hk, hw = _weight(hidden_w, (D,))
    pk, pw = _weight(pre_w, (L, D))
    out = np.empty((L, T, D), dtype=np.uint16)
    flags = (1 if hidden_input_scale else 0) | (2 if pre_input_scale else 0)
    st = lib().nrc_oracle_context_norms_ex(
        _ptr(x, ctypes.c_uint16), T, D, None if hw is None else hw.ctypes.data, hk,
        None if pw is None else pw.ctypes.data, pk, L, hidden_eps, pre_eps, hidden_center, pre_center, flags,
        _ptr(out, ctypes.c_uint16))
    _check(st, "context_norms_ex")
    return out


def hidden_norm(x, hidden_w, hidden_eps=1e-6, hidden_center=0.0, pre_eps=1e-6):
    """x [T, 8192] bf16 bits -> (h [T, 8192] bf16 bits, r [T] float32): the
    hidden norm's bf16 output and each row's layer-norm scale."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    assert x.shape == (T, D)
    hw = None if hidden_w is None else _c(hidden_w, np.uint16)
    h = np.empty((T, D), dtype=np.uint16)
    r = np.empty(T, dtype=np.float32)
    st = lib().nrc_oracle_hidden_norm(_ptr(x, ctypes.c_uint16), T, D, _ptr(hw, ctypes.c_uint16), hidden_eps,
                                      hidden_center, pre_eps, _ptr(h, ctypes.c_uint16), _ptr(r, ctypes.c_float))
    _check(st, "hidden_norm")
    return h, r


def kv_project(A, B):
    """A [L, T, D] bf16 bits, B [L, D, N] bf16 bits -> C [L, T, N] float32."""
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    L, T, Dd = A.shape
    assert B.shape[0] == L and B.shape[1] == Dd
    N = B.shape[2]
    C = np.empty((L, T, N), dtype=np.float32)
    st = lib().nrc_oracle_kv_project(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), _ptr(C, ctypes.c_float),
                                     L, T, Dd, N)
    _check(st, "kv_project")
    return C


def kv_project_nd(A, B):
    """A [L, T, D] bf16 bits, B [L, N, D] bf16 bits (the pages' weight
    storage) -> C [L, T, N] float32."""
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    L, T, Dd = A.shape
    assert B.shape[0] == L and B.shape[2] == Dd
    N = B.shape[1]
    C = np.empty((L, T, N), dtype=np.float32)
    st = lib().nrc_oracle_kv_project_nd(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                        _ptr(C, ctypes.c_float), L, T, Dd, N)
    _check(st, "kv_project_nd")
    return C


def knorm_rope_head(k, cs_row, eps=1e-6):
    k = _c(k, np.uint16)
    assert k.shape == (HEAD_DIM,)
    cs = None if cs_row is None else _c(cs_row, np.uint16)
    out = np.empty(HEAD_DIM, dtype=np.uint16)
    lib().nrc_oracle_knorm_rope_head(_ptr(k, ctypes.c_uint16), _ptr(cs, ctypes.c_uint16), eps,
                                     _ptr(out, ctypes.c_uint16))
    return out


def cache_offset(slot, block_size, H, h):
    return int(lib().nrc_oracle_cache_offset(int(slot), int(block_size), int(H), int(h)))


def context_kv_store(kv, H, positions, slots, cos_sin, caches, block_size, eps=1e-6):
    """In place on `caches` [L, num_blocks, H, block_size, 128] bf16 bits.

    kv [L, T, 2 H 64] bf16 bits; positions [T] int64; slots [L, rows] int64;
    cos_sin [max_position, 64] bf16 bits or None."""
    kv = _c(kv, np.uint16)
    L, T, N = kv.shape
    assert N == 2 * H * HEAD_DIM
    positions = _c(positions, np.int64)
    slots = _c(slots, np.int64)
    assert slots.ndim == 2 and slots.shape[0] == L
    rows = slots.shape[1]
    assert caches.flags.c_contiguous and caches.dtype == np.uint16
    num_blocks = caches.shape[1]
    assert caches.shape == (L, num_blocks, H, block_size, 2 * HEAD_DIM)
    cs = None if cos_sin is None else _c(cos_sin, np.uint16)
    max_pos = 0 if cs is None else cs.shape[0]
    st = lib().nrc_oracle_context_kv_store(
        _ptr(kv, ctypes.c_uint16), L, T, H, _ptr(positions, ctypes.c_int64), _ptr(slots, ctypes.c_int64), rows,
        _ptr(cs, ctypes.c_uint16), max_pos, _ptr(caches, ctypes.c_uint16), num_blocks, block_size, eps)
    _check(st, "context_kv_store")


def context_kv_store_ex(kv, H, positions, slots, cos_sin, caches, block_size, num_blocks, block_stride,
                        page_stride, head_stride, eps=1e-6):
    """The store with per-layer slot lists and strided cache views.

    slots: a list of L entries, each an int64 array [rows_l] (rows_l <= T) or
    None (that layer stores nothing). caches: a list of L flat uint16 arrays,
    updated in place; element (b, o, h, c) of layer l at b * block_stride +
    o * page_stride + h * head_stride + c (K in c < 64, V in 64 <= c < 128)."""
    kv = _c(kv, np.uint16)
    L, T, N = kv.shape
    assert N == 2 * H * HEAD_DIM and len(slots) == L and len(caches) == L
    positions = _c(positions, np.int64)
    keep = [None if s is None else _c(s, np.int64) for s in slots]
    sp = (ctypes.c_void_p * L)(*[None if s is None else s.ctypes.data for s in keep])
    rows = np.array([0 if s is None else s.shape[0] for s in keep], dtype=np.int64)
    for c in caches:
        assert c.dtype == np.uint16 and c.ndim == 1 and c.flags.c_contiguous
    cp = (ctypes.c_void_p * L)(*[c.ctypes.data for c in caches])
    clen = np.array([c.shape[0] for c in caches], dtype=np.int64)
    cs = None if cos_sin is None else _c(cos_sin, np.uint16)
    max_pos = 0 if cs is None else cs.shape[0]
    st = lib().nrc_oracle_context_kv_store_ex(
        _ptr(kv, ctypes.c_uint16), L, T, H, _ptr(positions, ctypes.c_int64), sp, _ptr(rows, ctypes.c_int64),
        _ptr(cs, ctypes.c_uint16), max_pos, cp, _ptr(clen, ctypes.c_int64), num_blocks, block_size, block_stride,
        page_stride, head_stride, eps)
    _check(st, "context_kv_store_ex")


def f16_to_f32(h):
    return np.float32(lib().nrc_oracle_f16_to_f32(int(h)))


def _bweight(w, kind):
    """(kind code, array) of a boundary norm weight: None; uint16 bf16 bits
    (kind 'bf16') or f16 bits (kind 'f16'); float32."""
    if w is None:
        return 0, None
    w = np.ascontiguousarray(w)
    assert w.shape == (D,)
    if w.dtype == np.float32:
        return 2, w
    assert w.dtype == np.uint16
    return (3 if kind == "f16" else 1), w


def draft_boundary(branch, stream, alpha, beta, post_w=None, pre_w=None, post_eps=1e-6, pre_eps=1e-6,
                   post_center=0.0, pre_center=0.0, post_input_scale=False, pre_input_scale=False,
                   post_kind="bf16", pre_kind="bf16", store_stream=True):
    """The residual boundary. branch [m, 8192] bf16 bits; stream [m, 8192]
    float32 or bf16 bits (uint16); alpha, beta float32 [8192]; weights None,
    float32, or uint16 bits read as bf16 or f16 (post_kind / pre_kind).
    Returns (new stream float32 or None, out bf16 bits)."""
    branch = _c(branch, np.uint16)
    m = branch.shape[0]
    assert branch.shape == (m, D)
    stream = np.ascontiguousarray(stream)
    assert stream.shape == (m, D) and stream.dtype in (np.float32, np.uint16)
    sk = 0 if stream.dtype == np.float32 else 1
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    pk, pw = _bweight(post_w, post_kind)
    qk, qw = _bweight(pre_w, pre_kind)
    out = np.empty((m, D), dtype=np.uint16)
    new = np.empty((m, D), dtype=np.float32) if store_stream else None
    flags = (1 if post_input_scale else 0) | (2 if pre_input_scale else 0)
    st = lib().nrc_oracle_draft_boundary(
        _ptr(branch, ctypes.c_uint16), m, stream.ctypes.data, sk, _ptr(alpha, ctypes.c_float),
        _ptr(beta, ctypes.c_float), None if pw is None else pw.ctypes.data, pk,
        None if qw is None else qw.ctypes.data, qk, post_eps, pre_eps, post_center, pre_center, flags,
        _ptr(new, ctypes.c_float), _ptr(out, ctypes.c_uint16))
    _check(st, "draft_boundary")
    return new, out


def chain(x, hidden_w, pre_w, L, w_kv, H, positions, slots, cos_sin, caches, block_size,
          hidden_eps=1e-6, pre_eps=1e-6, k_eps=1e-6):
    """The whole chain on the CPU; caches updated in place. Returns (normed, kv)."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    N = 2 * H * HEAD_DIM
    w_kv = _c(w_kv, np.uint16)
    assert w_kv.shape == (L, D, N)
    hw = None if hidden_w is None else _c(hidden_w, np.uint16)
    pw = None if pre_w is None else _c(pre_w, np.uint16)
    positions = _c(positions, np.int64)
    slots = _c(slots, np.int64)
    rows = slots.shape[1]
    num_blocks = caches.shape[1]
    cs = None if cos_sin is None else _c(cos_sin, np.uint16)
    max_pos = 0 if cs is None else cs.shape[0]
    normed = np.empty((L, T, D), dtype=np.uint16)
    kv = np.empty((L, T, N), dtype=np.uint16)
    st = lib().nrc_oracle_chain(
        _ptr(x, ctypes.c_uint16), T, _ptr(hw, ctypes.c_uint16), _ptr(pw, ctypes.c_uint16), L, hidden_eps, pre_eps,
        _ptr(w_kv, ctypes.c_uint16), H, _ptr(positions, ctypes.c_int64), _ptr(slots, ctypes.c_int64), rows,
        _ptr(cs, ctypes.c_uint16), max_pos, _ptr(caches, ctypes.c_uint16), num_blocks, block_size, k_eps,
        _ptr(normed, ctypes.c_uint16), _ptr(kv, ctypes.c_uint16))
    _check(st, "chain")
    return normed, kv
