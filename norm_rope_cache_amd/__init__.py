"""norm_rope_cache_amd: the DSpark draft's context K/V chain on MI355X (gfx950).

A thin ctypes binding over libnrc.so (include/nrc.h). Each function checks
torch tensor dtypes/shapes, passes raw device pointers and the current HIP
stream, and raises NrcError on a non-zero status. Every step of the chain
runs in the library's HIP kernels; there is no CPU or PyTorch fallback: if
libnrc.so is missing, every call raises.

    context_norms(x, hidden_w, pre_w, L, ...)      -> [L, T, 8192] bf16
    context_norms_ex(...)                          the same with FP32 / input-scaled weights
    context_kv_project(normed, w_kv)               -> [L, T, N] bf16 ([L, D, N] or [L, N, D] weights)
    context_kv_store(kv, positions, slots, cos_sin, caches, H, ...)   (in place)
    context_kv_store_ex(...)                       per-layer slot lists, strided cache views
    context_hidden_norm(x, ...) -> (h, r)          pre-pass of the fused path
    context_kv_project_fused(h, r, pre_w, w_kv)    projection with the layer norms fused in
    context_kv_chain(...)                          the whole chain (unfused by default)
    draft_boundary(branch, stream_in, alpha, beta, ...)   the residual boundary
"""

import ctypes
import os

__all__ = [
    "NrcError",
    "context_norms",
    "context_norms_ex",
    "context_kv_project",
    "context_kv_store",
    "context_kv_store_ex",
    "draft_boundary",
    "context_kv_chain",
    "context_hidden_norm",
    "context_kv_project_fused",
    "context_kv_project_noalloc",
    "kv_views",
    "check_scalars",
    "check_bf16_pair",
    "library_path",
    "abi_version",
]

HIDDEN = 8192
HEAD_DIM = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnrc.so")
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class NrcError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"libnrc status {code}: {message}")
        self.code = code


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libnrc.so not built at {_LIB_PATH}: run `python -m norm_rope_cache_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(_LIB_PATH)
    L.nrc_last_error.restype = ctypes.c_char_p
    L.nrc_last_error.argtypes = []
    L.nrc_abi_version.restype = _i32
    L.nrc_abi_version.argtypes = []
    L.nrc_context_norms.restype = _i32
    L.nrc_context_norms.argtypes = [_vp, _i64, _i64, _vp, _vp, _i32, _f32, _f32, _f32, _f32, _vp, _vp]
    L.nrc_context_norms_ex.restype = _i32
    L.nrc_context_norms_ex.argtypes = [_vp, _i64, _i64, _vp, _i32, _vp, _i32, _i32, _f32, _f32, _f32, _f32,
                                       ctypes.c_uint32, _vp, _vp]
    L.nrc_context_kv_store_ex.restype = _i32
    L.nrc_context_kv_store_ex.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                          _i64, _i64, _i64, _i64, _i64, _i32, _i32, _f32, _vp]
    L.nrc_context_kv_project_ex.restype = _i32
    L.nrc_context_kv_project_ex.argtypes = [_vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp]
    L.nrc_draft_boundary.restype = _i32
    L.nrc_draft_boundary.argtypes = [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _f32, _f32, _f32,
                                     _f32, ctypes.c_uint32, _vp, _vp, _vp]
    L.nrc_context_kv_project.restype = _i32
    L.nrc_context_kv_project.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp]
    L.nrc_context_kv_project_workspace_bytes.restype = _i64
    L.nrc_context_kv_project_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64]
    L.nrc_context_kv_project_split.restype = _i32
    L.nrc_context_kv_project_split.argtypes = [_vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp]
    L.nrc_context_kv_project_noalloc.restype = _i32
    L.nrc_context_kv_project_noalloc.argtypes = [_vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp]
    L.nrc_context_kv_project_timed.restype = _i32
    L.nrc_context_kv_project_timed.argtypes = [_vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp,
                                               _vp]
    L.nrc_context_kv_store.restype = _i32
    L.nrc_context_kv_store.argtypes = [
        _vp, _vp, _i64, _i64, _i64, _i64, _vp, ctypes.POINTER(_vp), _i64, _i64, _vp, _i64,
        ctypes.POINTER(_vp), _i64, _i64, _i32, _i32, _f32, _vp]
    L.nrc_context_kv_project_store.restype = _i32
    L.nrc_context_kv_project_store.argtypes = [
        _vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, ctypes.POINTER(_vp), _i64, _vp, _i64,
        ctypes.POINTER(_vp), _i64, _i64, _f32, _vp]
    L.nrc_context_hidden_norm.restype = _i32
    L.nrc_context_hidden_norm.argtypes = [_vp, _i64, _i64, _vp, _vp, _i32, _f32, _f32, _f32, _f32, _vp, _vp, _vp]
    L.nrc_context_kv_project_fused.restype = _i32
    L.nrc_context_kv_project_fused.argtypes = [_vp, _vp, _vp, _f32, _vp, _vp, _i32, _i64, _i64, _i64, _vp]
    L.nrc_context_kv_project_fused_split.restype = _i32
    L.nrc_context_kv_project_fused_split.argtypes = [_vp, _vp, _vp, _f32, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i64,
                                                     _vp]
    L.nrc_check_scalars.restype = _i32
    L.nrc_check_scalars.argtypes = [_vp, _vp, _vp, _i64, _vp]
    L.nrc_traffic_twin.restype = _i32
    L.nrc_traffic_twin.argtypes = [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _i64, _vp]
    L.nrc_check_bf16_pair.restype = _i32
    L.nrc_check_bf16_pair.argtypes = [_vp, _vp, _i64, _vp]
    _lib = L
    return L


def abi_version():
    return int(_load().nrc_abi_version())


def _check(code):
    if code != 0:
        msg = _load().nrc_last_error().decode(errors="replace")
        raise NrcError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref):
    """The HIP stream for a call on ref's GPU: the given torch stream, which
    must belong to that GPU, or that GPU's current stream."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    elif stream.device != ref.device:
        raise ValueError(f"stream is on {stream.device}, the operands on {ref.device}")
    return ctypes.c_void_p(stream.cuda_stream)


def _call(ref, fn, *args):
    """One C-ABI call with ref's GPU as the current device (the library sizes
    its launches and finds its scratch on the current device), raising
    NrcError on a non-zero status."""
    import torch

    dev = ref.device.index
    if dev is not None and dev != torch.cuda.current_device():
        with torch.cuda.device(dev):
            _check(fn(*args))
    else:
        _check(fn(*args))


def _all_on(ref, **tensors):
    """_same_device for every operand given (None: absent)."""
    for name, t in tensors.items():
        if t is not None:
            _same_device(t, ref, name)


def _bf16(t, name, contiguous=True):
    import torch

    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, not {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(t, ref, name):
    """Raise unless t is a tensor on ref's GPU: a host pointer handed to a
    kernel would fault the device instead of failing."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != ref.device:
        where = "not a tensor" if not isinstance(t, torch.Tensor) else str(t.device)
        raise ValueError(f"{name} must be a tensor on {ref.device} ({where})")
    return t


def context_norms(x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, hidden_center=0.0, pre_center=0.0,
                  out=None, stream=None):
    """stack([pre_norm_l(hidden_norm(x)) for l]): x [T, 8192] bf16 ->
    [L, T, 8192] bf16 (written into `out` when given)."""
    import torch

    _bf16(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, 8192]")
    T, D = x.shape
    if hidden_w is not None:
        _bf16(hidden_w, "hidden_w")
        if tuple(hidden_w.shape) != (D,):
            raise ValueError("hidden_w must be [D]")
    if pre_w is not None:
        _bf16(pre_w, "pre_w")
        if tuple(pre_w.shape) != (L, D):
            raise ValueError("pre_w must be [L, D]")
    if out is None:
        out = torch.empty((L, T, D), dtype=torch.bfloat16, device=x.device)
    else:
        _bf16(out, "out")
        if tuple(out.shape) != (L, T, D):
            raise ValueError("out must be [L, T, D]")
    _all_on(x, hidden_w=hidden_w, pre_w=pre_w, out=out)
    _call(x, _load().nrc_context_norms, _ptr(x), T, D, _ptr(hidden_w), _ptr(pre_w), L, hidden_eps, pre_eps,
          hidden_center, pre_center, _ptr(out), _stream(stream, x))
    return out


WEIGHT_NONE, WEIGHT_BF16, WEIGHT_F32 = 0, 1, 2
HIDDEN_INPUT_SCALE, PRE_INPUT_SCALE = 1, 2


def _weight_kind(w, name, shape):
    import torch

    if w is None:
        return WEIGHT_NONE
    if not w.is_cuda or not w.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(w.shape) != shape:
        raise ValueError(f"{name} must be {list(shape)}")
    if w.dtype == torch.bfloat16:
        return WEIGHT_BF16
    if w.dtype == torch.float32:
        return WEIGHT_F32
    raise ValueError(f"{name} must be bf16 or float32, not {w.dtype}")


def context_norms_ex(x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, hidden_center=0.0, pre_center=0.0,
                     hidden_input_scale=False, pre_input_scale=False, out=None, stream=None):
    """context_norms with bf16 or float32 weights and, per norm, the weight
    scaling the norm's input instead of its output."""
    import torch

    _bf16(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, 8192]")
    T, D = x.shape
    hk = _weight_kind(hidden_w, "hidden_w", (D,))
    pk = _weight_kind(pre_w, "pre_w", (L, D))
    if out is None:
        out = torch.empty((L, T, D), dtype=torch.bfloat16, device=x.device)
    else:
        _bf16(out, "out")
        if tuple(out.shape) != (L, T, D):
            raise ValueError("out must be [L, T, D]")
    _all_on(x, hidden_w=hidden_w, pre_w=pre_w, out=out)
    flags = (HIDDEN_INPUT_SCALE if hidden_input_scale else 0) | (PRE_INPUT_SCALE if pre_input_scale else 0)
    _call(x, _load().nrc_context_norms_ex, _ptr(x), T, D, _ptr(hidden_w), hk, _ptr(pre_w), pk, L, hidden_eps, pre_eps,
          hidden_center, pre_center, flags, _ptr(out), _stream(stream, x))
    return out


def _boundary_kind(w, name):
    import torch

    if w is None:
        return WEIGHT_NONE
    if not w.is_cuda or not w.is_contiguous() or tuple(w.shape) != (8192,):
        raise ValueError(f"{name} must be a contiguous device tensor of shape [8192]")
    kinds = {torch.bfloat16: WEIGHT_BF16, torch.float32: WEIGHT_F32, torch.float16: 3}
    if w.dtype not in kinds:
        raise ValueError(f"{name} must be bf16, float32 or float16, not {w.dtype}")
    return kinds[w.dtype]


def draft_boundary(branch, stream_in, alpha, beta, post_w=None, pre_w=None, post_eps=1e-6, pre_eps=1e-6,
                   post_center=0.0, pre_center=0.0, post_input_scale=False, pre_input_scale=False,
                   store_stream=True, out=None, stream_out=None, stream=None):
    """One residual boundary: (new FP32 stream or None, bf16 out [m, 8192]).

    branch [m, 8192] bf16; stream_in [m, 8192] float32 or bf16; alpha, beta
    float32 [8192]; post_w / pre_w [8192] bf16, float32 or float16 (None:
    weightless); *_input_scale: that weight scales the norm's input."""
    import torch

    _bf16(branch, "branch")
    if branch.dim() != 2:
        raise ValueError("branch must be [m, 8192]")
    m, D = branch.shape
    if tuple(stream_in.shape) != (m, D) or not stream_in.is_contiguous() or not stream_in.is_cuda:
        raise ValueError("stream_in must be a contiguous device tensor shaped like the branch")
    if stream_in.dtype == torch.float32:
        sk = 0
    elif stream_in.dtype == torch.bfloat16:
        sk = 1
    else:
        raise ValueError("stream_in must be float32 or bf16")
    for g, name in ((alpha, "alpha"), (beta, "beta")):
        if g.dtype != torch.float32 or tuple(g.shape) != (D,) or not g.is_contiguous() or not g.is_cuda:
            raise ValueError(f"{name} must be a contiguous float32 device tensor [8192]")
    pk = _boundary_kind(post_w, "post_w")
    qk = _boundary_kind(pre_w, "pre_w")
    if out is None:
        out = torch.empty((m, D), dtype=torch.bfloat16, device=branch.device)
    else:
        _bf16(out, "out")
        if tuple(out.shape) != (m, D):
            raise ValueError("out must be [m, 8192] like the branch")
    if not store_stream:
        stream_out = None
    elif stream_out is None:
        stream_out = torch.empty((m, D), dtype=torch.float32, device=branch.device)
    elif stream_out.dtype != torch.float32 or tuple(stream_out.shape) != (m, D) or not stream_out.is_contiguous():
        raise ValueError("stream_out must be a contiguous float32 [m, 8192] tensor")
    _all_on(branch, stream_in=stream_in, alpha=alpha, beta=beta, post_w=post_w, pre_w=pre_w, out=out,
            stream_out=stream_out)
    flags = (1 if post_input_scale else 0) | (2 if pre_input_scale else 0)
    _call(branch, _load().nrc_draft_boundary, _ptr(branch), m, D, _ptr(stream_in), sk, _ptr(alpha), _ptr(beta),
          _ptr(post_w), pk, _ptr(pre_w), qk, post_eps, pre_eps, post_center, pre_center, flags, _ptr(stream_out),
          _ptr(out), _stream(stream, branch))
    return stream_out, out


def context_hidden_norm(x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, hidden_center=0.0, pre_center=0.0,
                        h=None, r=None, stream=None):
    """Pre-pass of the fused path: (h [T, 8192] bf16, r [T] float32)."""
    import torch

    _bf16(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, 8192]")
    T, D = x.shape
    if hidden_w is not None:
        _bf16(hidden_w, "hidden_w")
        if tuple(hidden_w.shape) != (D,):
            raise ValueError("hidden_w must be [D]")
    if pre_w is not None:
        _bf16(pre_w, "pre_w")
        if tuple(pre_w.shape) != (L, D):
            raise ValueError("pre_w must be [L, D]")
    _all_on(x, hidden_w=hidden_w, pre_w=pre_w)
    if h is None:
        h = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if r is None:
        r = torch.empty((T,), dtype=torch.float32, device=x.device)
    _bf16(h, "h")
    if tuple(h.shape) != (T, D) or r.dtype != torch.float32 or tuple(r.shape) != (T,) or not r.is_contiguous():
        raise ValueError("h must be [T, D] bf16 and r [T] float32")
    _same_device(h, x, "h")
    _same_device(r, x, "r")
    _call(x, _load().nrc_context_hidden_norm, _ptr(x), T, D, _ptr(hidden_w), _ptr(pre_w), L, hidden_eps, pre_eps,
          hidden_center, pre_center, _ptr(h), _ptr(r), _stream(stream, x))
    return h, r


def context_kv_project_fused(h, r, pre_w, w_kv, pre_center=0.0, out=None, stream=None, split=True):
    """kv[l] = bf16((h * |r|) * (pre_w[l] + pre_center)) . w_kv[l]; equal to
    context_norms followed by context_kv_project with the same `split`
    (small T: the summation split over several workgroups, with a workspace
    from torch's allocator; split=False keeps the one-pass kernel)."""
    import torch

    _bf16(h, "h")
    _bf16(w_kv, "w_kv")
    if h.dim() != 2 or w_kv.dim() != 3:
        raise ValueError("h must be [T, D] and w_kv [L, D, N]")
    T, D = h.shape
    L, Dw, N = w_kv.shape
    if Dw != D:
        raise ValueError("w_kv must be [L, D, N]")
    if pre_w is not None:
        _bf16(pre_w, "pre_w")
        if tuple(pre_w.shape) != (L, D):
            raise ValueError("pre_w must be [L, D]")
    if r.dtype != torch.float32 or tuple(r.shape) != (T,) or not r.is_contiguous():
        raise ValueError("r must be a contiguous float32 [T]")
    _same_device(r, h, "r")
    _same_device(w_kv, h, "w_kv")
    if pre_w is not None:
        _same_device(pre_w, h, "pre_w")
    if out is None:
        out = torch.empty((L, T, N), dtype=torch.bfloat16, device=h.device)
    else:
        _bf16(out, "out")
        _same_device(out, h, "out")
        if tuple(out.shape) != (L, T, N):
            raise ValueError("out must be [L, T, N]")
    lib = _load()
    need = lib.nrc_context_kv_project_workspace_bytes(L, T, D, N) if split else 0
    if need < 0:
        _check(need)
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=h.device)
        if stream is not None:
            ws.record_stream(stream)  # the allocator may reuse it only after this stream's work
        _call(h, lib.nrc_context_kv_project_fused_split, _ptr(h), _ptr(r), _ptr(pre_w), pre_center, _ptr(w_kv),
              _ptr(out), L, T, D, N, _ptr(ws), need, _stream(stream, h))
    else:
        _call(h, lib.nrc_context_kv_project_fused, _ptr(h), _ptr(r), _ptr(pre_w), pre_center, _ptr(w_kv), _ptr(out), L,
              T, D, N, _stream(stream, h))
    return out


def _project_operands(normed, w_kv, out, w_layout):
    """Shape checks of the projection; returns L, T, D, N, the layout code and out."""
    import torch

    _bf16(normed, "normed")
    _bf16(w_kv, "w_kv")
    _same_device(w_kv, normed, "w_kv")
    if normed.dim() != 3:
        raise ValueError("normed must be [L, T, D]")
    L, T, D = normed.shape
    if w_layout == "dn":
        if w_kv.dim() != 3 or w_kv.shape[0] != L or w_kv.shape[1] != D:
            raise ValueError("w_kv must be [L, D, N]")
        N = w_kv.shape[2]
    elif w_layout == "nd":
        if w_kv.dim() != 3 or w_kv.shape[0] != L or w_kv.shape[2] != D:
            raise ValueError("w_kv must be [L, N, D]")
        N = w_kv.shape[1]
    else:
        raise ValueError("w_layout is 'dn' or 'nd'")
    if out is None:
        out = torch.empty((L, T, N), dtype=torch.bfloat16, device=normed.device)
    else:
        _bf16(out, "out")
        _same_device(out, normed, "out")
        if tuple(out.shape) != (L, T, N):
            raise ValueError("out must be [L, T, N]")
    return L, T, D, N, (0 if w_layout == "dn" else 1), out


def context_kv_project(normed, w_kv, out=None, stream=None, w_layout="dn", split=True):
    """[L, T, D] x [L, D, N] -> [L, T, N] bf16 (FP32 accumulation).
    w_layout "nd": w_kv is stored [L, N, D] (the pages' storage). split: for
    shapes with too few output tiles to fill the GPU (small T) the summation
    axis is split over several workgroups, with a workspace from torch's
    allocator (split=False keeps the one-pass kernel)."""
    import torch

    L, T, D, N, layout, out = _project_operands(normed, w_kv, out, w_layout)
    lib = _load()
    need = lib.nrc_context_kv_project_workspace_bytes(L, T, D, N) if split else 0
    if need < 0:
        _check(need)
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=normed.device)
        if stream is not None:
            ws.record_stream(stream)  # the allocator may reuse it only after this stream's work
        _call(normed, lib.nrc_context_kv_project_split, _ptr(normed), _ptr(w_kv), layout, _ptr(out), L, T, D, N,
              _ptr(ws), need, _stream(stream, normed))
    elif w_layout == "dn":
        _call(normed, lib.nrc_context_kv_project, _ptr(normed), _ptr(w_kv), _ptr(out), L, T, D, N,
              _stream(stream, normed))
    else:
        _call(normed, lib.nrc_context_kv_project_ex, _ptr(normed), _ptr(w_kv), 1, _ptr(out), L, T, D, N,
              _stream(stream, normed))
    return out


def context_kv_project_noalloc(normed, w_kv, out, stream=None, w_layout="dn"):
    """context_kv_project for callers that cannot allocate: the split form's
    partial sums go to the library's per-GPU scratch (no workspace, no
    allocation by the library or here; `out` is required). Same bits as
    context_kv_project; raises NrcError for a split needing more scratch
    than the library holds. Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("context_kv_project_noalloc writes into a caller-owned out")
    L, T, D, N, layout, out = _project_operands(normed, w_kv, out, w_layout)
    _call(normed, _load().nrc_context_kv_project_noalloc, _ptr(normed), _ptr(w_kv), layout, _ptr(out), L, T, D, N,
          _stream(stream, normed))
    return out


def context_kv_project_timed(normed, w_kv, out=None, stream=None, w_layout="dn"):
    """The one-pass projection with per-workgroup clock stamps (a diagnostic;
    the call synchronizes the device to read them). Returns (out, clocks):
    clocks holds 'workgroups', 'stamps' (CPU int64 [workgroups, 4]: shader
    clock at start, constant clock at start, shader clock at end, constant
    clock at end), 'wall_khz' (the constant clock's rate) and 'shader_ghz'
    (each workgroup's mean shader clock over its lifetime, GHz)."""
    import ctypes
    import torch

    L, T, D, N, layout, out = _project_operands(normed, w_kv, out, w_layout)
    lib = _load()
    n = 8 * torch.cuda.get_device_properties(normed.device).multi_processor_count
    stamps = torch.zeros(n, dtype=torch.int64, device=normed.device)
    wg, khz = ctypes.c_int32(0), ctypes.c_int32(0)
    _call(normed, lib.nrc_context_kv_project_timed, _ptr(normed), _ptr(w_kv), layout, _ptr(out), L, T, D, N,
          _ptr(stamps), n, ctypes.byref(wg), ctypes.byref(khz), _stream(stream, normed))
    torch.cuda.synchronize(normed.device)
    st = stamps[: 4 * wg.value].view(-1, 4).cpu()
    ds = (st[:, 2] - st[:, 0]).double()
    dr = (st[:, 3] - st[:, 1]).double()
    ghz = (ds / dr * khz.value / 1e6) if wg.value else torch.empty(0, dtype=torch.float64)
    return out, {"workgroups": wg.value, "stamps": st, "wall_khz": khz.value, "shader_ghz": ghz}


def kv_views(kv, H):
    """k, v views [L, T, H, 64] of a projection output [L, T, 2 H 64]."""
    L, T, N = kv.shape
    v5 = kv.view(L, T, 2, H, HEAD_DIM)
    return v5[:, :, 0], v5[:, :, 1]


def _store_operands(kv_ref, L, T, H, positions, slots, cos_sin, caches, rows):
    """Checks of the store's operands against the K/V source kv_ref ([L, T, ...]
    on one device); returns the host pointer arrays and sizes the C ABI takes:
    (slot_arr, cache_arr, n_rows, num_blocks, block_size, max_position)."""
    import torch

    # Per-layer pointers: a contiguous stacked tensor is addressed by its
    # layer stride (no per-layer views); lists and other tensors layer by layer.
    if isinstance(caches, torch.Tensor) and caches.dim() == 5 and caches.is_contiguous():
        _bf16(caches, "cache")
        _same_device(caches, kv_ref, "caches")
        if caches.shape[0] != L:
            raise ValueError("one cache and one slot mapping per layer")
        if caches.shape[2] != H or caches.shape[4] != 2 * HEAD_DIM:
            raise ValueError("caches must be [num_blocks, H, block_size, 128]")
        nb, bs = caches.shape[1], caches.shape[3]
        c_base, c_step = caches.data_ptr(), caches.stride(0) * 2
        cache_ptrs = [c_base + i * c_step for i in range(L)]
    else:
        cache_list = list(caches) if not isinstance(caches, torch.Tensor) else [caches[i] for i in range(caches.shape[0])]
        if len(cache_list) != L:
            raise ValueError("one cache and one slot mapping per layer")
        c0 = cache_list[0]
        if c0.dim() != 4 or c0.shape[1] != H or c0.shape[3] != 2 * HEAD_DIM:
            raise ValueError("caches must be [num_blocks, H, block_size, 128]")
        nb, _, bs, _ = c0.shape
        for c in cache_list:
            _bf16(c, "cache")
            _same_device(c, kv_ref, "caches")
            if c.shape != c0.shape:
                raise ValueError("all caches must have one shape")
        cache_ptrs = [c.data_ptr() for c in cache_list]
    if isinstance(slots, torch.Tensor) and slots.dim() == 1:
        # one mapping shared by every layer: each layer's pointer is the same array
        if slots.dtype != torch.int64 or not slots.is_contiguous():
            raise ValueError("slots must be contiguous int64 [rows] tensors of one length")
        _same_device(slots, kv_ref, "slots")
        slot_len = slots.shape[0]
        slot_ptrs = [slots.data_ptr()] * L
    elif isinstance(slots, torch.Tensor) and slots.dim() == 2 and slots.is_contiguous():
        if slots.dtype != torch.int64:
            raise ValueError("slots must be contiguous int64 [rows] tensors of one length")
        if slots.shape[0] != L:
            raise ValueError("one cache and one slot mapping per layer")
        _same_device(slots, kv_ref, "slots")
        slot_len = slots.shape[1]
        s_base, s_step = slots.data_ptr(), slots.stride(0) * 8
        slot_ptrs = [s_base + i * s_step for i in range(L)]
    else:
        slot_list = list(slots) if not isinstance(slots, torch.Tensor) else [slots[i] for i in range(slots.shape[0])]
        if len(slot_list) != L:
            raise ValueError("one cache and one slot mapping per layer")
        for s in slot_list:
            if (not isinstance(s, torch.Tensor) or s.dtype != torch.int64 or s.dim() != 1 or not s.is_contiguous()
                    or s.shape[0] != slot_list[0].shape[0]):
                raise ValueError("slots must be contiguous int64 [rows] tensors of one length")
            _same_device(s, kv_ref, "slots")
        slot_len = slot_list[0].shape[0]
        slot_ptrs = [s.data_ptr() for s in slot_list]
    n_rows = slot_len if rows is None else int(rows)
    if n_rows < 0 or n_rows > slot_len:
        raise ValueError(f"rows = {n_rows} must lie in [0, {slot_len}] (the slot mapping's length)")
    if n_rows > T:
        raise ValueError(f"rows = {n_rows} exceeds the {T} rows of kv")
    if cos_sin is not None:
        _bf16(cos_sin, "cos_sin")
        _same_device(cos_sin, kv_ref, "cos_sin")
        if cos_sin.dim() != 2 or cos_sin.shape[1] != HEAD_DIM:
            raise ValueError("cos_sin must be [max_position, 64]")
        if positions is None or positions.dtype != torch.int64 or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int64 tensor")
        _same_device(positions, kv_ref, "positions")
        if positions.shape[0] < n_rows:
            raise ValueError("positions shorter than the inserted rows")
    slot_arr = (_vp * L)(*slot_ptrs)
    cache_arr = (_vp * L)(*cache_ptrs)
    max_pos = 0 if cos_sin is None else cos_sin.shape[0]
    return slot_arr, cache_arr, n_rows, nb, bs, max_pos


def context_kv_store_ex(kv, positions, slots, cos_sin, caches, H, eps=1e-6, k=None, v=None, stream=None):
    """The store with per-layer slot lists and strided cache views, in place.

    slots   a list of L entries: a contiguous int64 [rows_l] tensor (its
            first rows_l rows are inserted) or None (the layer stores nothing)
    caches  a list of L [num_blocks, H, block_size, 128] bf16 views of one
            shape and stride, unit last stride (any block / head / page
            strides that are multiples of 8), or None where slots is None
    Other arguments as context_kv_store."""
    import torch

    if k is None:
        _bf16(kv, "kv")
        k, v = kv_views(kv, H)
    for name, t in (("k", k), ("v", v)):
        _bf16(t, name, contiguous=False)
        if t.dim() != 4 or t.shape[2] != H or t.shape[3] != HEAD_DIM or t.stride(3) != 1 or t.stride(2) != HEAD_DIM:
            raise ValueError(f"{name} must be an [L, T, H, 64] view with unit last stride and head stride 64")
    L, T = k.shape[0], k.shape[1]
    _same_device(v, k, "v")
    slot_list, cache_list = list(slots), list(caches)
    if len(slot_list) != L or len(cache_list) != L:
        raise ValueError("one cache and one slot list (or None) per layer")
    live = [c for s, c in zip(slot_list, cache_list) if s is not None]
    if not live:
        return
    c0 = live[0]
    if c0.dim() != 4 or c0.shape[1] != H or c0.shape[3] != 2 * HEAD_DIM or c0.stride(3) != 1:
        raise ValueError("caches must be [num_blocks, H, block_size, 128] views with unit last stride")
    for c in live:
        if c is None or c.dtype != torch.bfloat16 or not c.is_cuda:
            raise ValueError("every layer with slots needs a bf16 device cache")
        _same_device(c, k, "caches")
        if c.shape != c0.shape or c.stride() != c0.stride():
            raise ValueError("all caches must have one shape and one stride")
    nb, _, bs, _ = c0.shape
    rows = []
    for s in slot_list:
        if s is None:
            rows.append(0)
            continue
        if not isinstance(s, torch.Tensor) or s.dtype != torch.int64 or s.dim() != 1 or not s.is_contiguous():
            raise ValueError("slots must be contiguous int64 [rows] tensors")
        _same_device(s, k, "slots")
        rows.append(s.shape[0])
    if cos_sin is not None:
        _bf16(cos_sin, "cos_sin")
        _same_device(cos_sin, k, "cos_sin")
        if cos_sin.dim() != 2 or cos_sin.shape[1] != HEAD_DIM:
            raise ValueError("cos_sin must be [max_position, 64]")
        if positions is None or positions.dtype != torch.int64 or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int64 tensor")
        _same_device(positions, k, "positions")
        if positions.shape[0] < max(rows):
            raise ValueError("positions shorter than the inserted rows")
    slot_arr = (_vp * L)(*[None if s is None else s.data_ptr() for s in slot_list])
    cache_arr = (_vp * L)(*[None if (s is None or c is None) else c.data_ptr()
                            for s, c in zip(slot_list, cache_list)])
    row_arr = (ctypes.c_int64 * L)(*rows)
    max_pos = 0 if cos_sin is None else cos_sin.shape[0]
    _call(k, _load().nrc_context_kv_store_ex, _ptr(k), _ptr(v), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
          _ptr(positions) if cos_sin is not None else None, slot_arr, row_arr, T, _ptr(cos_sin), max_pos, cache_arr, nb,
          bs, c0.stride(0), c0.stride(2), c0.stride(1), H, L, eps, _stream(stream, k))


def context_kv_store(kv, positions, slots, cos_sin, caches, H, eps=1e-6, rows=None, k=None, v=None,
                     stream=None):
    """K-norm + GPT-J RoPE + paged insert, in place on `caches`.

    kv       [L, T, 2 H 64] bf16 projection output (or pass k, v views
             [L, T, H, 64] with unit last stride and head stride 64)
    positions [T] int64 (unused without cos_sin)
    slots    [rows] int64 tensor (one mapping shared by every layer), an
             [L, rows] int64 tensor or a list of L [rows] int64 tensors
    rows     the first `rows` rows are inserted (default: the mapping's
             length; at most that length and T)
    cos_sin  [max_position, 64] bf16 or None (RoPE off)
    caches   [L, num_blocks, H, block_size, 128] bf16 tensor or a list of L
             [num_blocks, H, block_size, 128] tensors
    """
    import torch

    if k is None:
        _bf16(kv, "kv")
        if kv.dim() != 3 or kv.shape[2] != 2 * H * HEAD_DIM:
            raise ValueError("kv must be [L, T, 2 H 64]")
        # K and V are the two halves of each contiguous kv row
        L, T = kv.shape[0], kv.shape[1]
        k_ptr = kv.data_ptr()
        v_ptr = k_ptr + H * HEAD_DIM * 2
        k_ls = v_ls = kv.stride(0)
        k_rs = v_rs = kv.stride(1)
    else:
        for name, t in (("k", k), ("v", v)):
            _bf16(t, name, contiguous=False)
            if t.dim() != 4 or t.shape[2] != H or t.shape[3] != HEAD_DIM or t.stride(3) != 1 or t.stride(2) != HEAD_DIM:
                raise ValueError(f"{name} must be an [L, T, H, 64] view with unit last stride and head stride 64")
        L, T = k.shape[0], k.shape[1]
        _same_device(v, k, "v")
        k_ptr, v_ptr = k.data_ptr(), v.data_ptr()
        k_ls, k_rs, v_ls, v_rs = k.stride(0), k.stride(1), v.stride(0), v.stride(1)
    kv_ref = kv if k is None else k
    slot_arr, cache_arr, n_rows, nb, bs, max_pos = _store_operands(kv_ref, L, T, H, positions, slots, cos_sin,
                                                                  caches, rows)
    _call(kv_ref, _load().nrc_context_kv_store, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), k_ls, k_rs, v_ls, v_rs,
          _ptr(positions) if cos_sin is not None else None, slot_arr, n_rows, T, _ptr(cos_sin), max_pos, cache_arr, nb,
          bs, H, L, eps, _stream(stream, kv_ref))


def context_kv_project_store(normed, w_kv, positions, slots, cos_sin, caches, eps=1e-6, rows=None, out=None,
                             stream=None, w_layout="dn"):
    """context_kv_project (split=True) then context_kv_store on its output,
    in one call: same kv and cache bits. Where the shape splits the
    summation (small T), the store's kernel adds the slices itself, writing
    kv and inserting each row in the same pass. H = N / 128. Returns kv."""
    import torch

    L, T, D, N, layout, out = _project_operands(normed, w_kv, out, w_layout)
    if N % (2 * HEAD_DIM):
        raise ValueError("N must be 2 H 64")
    H = N // (2 * HEAD_DIM)
    slot_arr, cache_arr, n_rows, nb, bs, max_pos = _store_operands(out, L, T, H, positions, slots, cos_sin, caches,
                                                                  rows)
    lib = _load()
    need = lib.nrc_context_kv_project_workspace_bytes(L, T, D, N)
    if need < 0:
        _check(need)
    ws = None
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=normed.device)
        if stream is not None:
            ws.record_stream(stream)
    _call(normed, lib.nrc_context_kv_project_store, _ptr(normed), _ptr(w_kv), layout, _ptr(out), L, T, D, N, _ptr(ws),
          need, _ptr(positions) if cos_sin is not None else None, slot_arr, n_rows, _ptr(cos_sin), max_pos, cache_arr,
          nb, bs, eps, _stream(stream, normed))
    return out


def check_scalars(x, want_bf16=True, want_rsqrt=True, stream=None):
    """Diagnostic: the library's device bf16 rounding and 1/sqrt applied to
    a float32 GPU tensor; returns (bf16 bits as int16 tensor, float32 tensor)."""
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 GPU tensor")
    bf = torch.empty(x.shape, dtype=torch.int16, device=x.device) if want_bf16 else None
    rs = torch.empty_like(x) if want_rsqrt else None
    _call(x, _load().nrc_check_scalars, _ptr(x), _ptr(bf), _ptr(rs), x.numel(), _stream(stream, x))
    return bf, rs


def check_bf16_pair(x, stream=None):
    """Diagnostic: the paired hardware bf16 conversion the norms use on
    NaN-free rows, applied to a float32 GPU tensor (bits as int16)."""
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 GPU tensor")
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    _call(x, _load().nrc_check_bf16_pair, _ptr(x), _ptr(out), x.numel(), _stream(stream, x))
    return out


TWIN_NORMS_STORES, TWIN_PLAIN_STORES, TWIN_READS_ONLY, TWIN_WRITES_ONLY = 0, 1, 2, 3


def traffic_twin(x, L, mode, out=None, per_cu=1, stream=None):
    """Diagnostic: the norms' HBM traffic (read x [T, 8192], write it to L
    rows of out [L, T, 8192]) in the norms' access pattern, no arithmetic;
    mode TWIN_* as in nrc.h. Returns out."""
    import torch

    _bf16(x, "x")
    T = x.shape[0]
    if tuple(x.shape) != (T, HIDDEN):
        raise ValueError("x must be [T, 8192]")
    if out is None and mode != TWIN_READS_ONLY:
        out = torch.empty((L, T, HIDDEN), dtype=torch.bfloat16, device=x.device)
    if out is not None:
        _bf16(out, "out")
        _same_device(out, x, "out")
        if tuple(out.shape) != (L, T, HIDDEN):
            raise ValueError("out must be [L, T, 8192]")
    sink = None
    if mode == TWIN_READS_ONLY:
        n = per_cu * torch.cuda.get_device_properties(x.device).multi_processor_count * 1024
        sink = torch.empty(n, dtype=torch.int32, device=x.device)
    _call(x, _load().nrc_traffic_twin, _ptr(x), T, L, mode, per_cu, _ptr(out), _ptr(sink),
          0 if sink is None else sink.numel(), _stream(stream, x))
    return out


def context_kv_chain(x, hidden_w, pre_w, w_kv, positions, slots, cos_sin, caches, H, hidden_eps=1e-6,
                     pre_eps=1e-6, k_eps=1e-6, fused=False, workspace=None, kv=None, stream=None, split=True):
    """The whole chain, in place on `caches`; returns kv [L, T, N].

    fused=False (the faster form on MI355X at H = 8): norms into `workspace`
    ([L, T, 8192] bf16) -> projection and store (one call with split=True). fused=True: pre-pass (h, r)
    -> fused projection -> store, without the [L, T, 8192] intermediate;
    `workspace` may be a tuple (h [T, 8192] bf16, r [T] float32). Both forms
    write the same bits for the same `split`; for small T split=True splits
    the summation (see context_kv_project), which changes the rounding
    within the projection's tolerance."""
    L = w_kv.shape[0]
    if fused:
        h, r = workspace if workspace is not None else (None, None)
        h, r = context_hidden_norm(x, hidden_w, pre_w, L, hidden_eps, pre_eps, h=h, r=r, stream=stream)
        kv = context_kv_project_fused(h, r, pre_w, w_kv, out=kv, stream=stream, split=split)
    else:
        normed = context_norms(x, hidden_w, pre_w, L, hidden_eps, pre_eps, out=workspace, stream=stream)
        if split:
            # the projection and the store in one call (same bits as the two)
            if w_kv.shape[2] != 2 * H * HEAD_DIM:
                raise ValueError("w_kv must be [L, D, 2 H 64]")
            return context_kv_project_store(normed, w_kv, positions, slots, cos_sin, caches, k_eps, out=kv,
                                            stream=stream)
        kv = context_kv_project(normed, w_kv, out=kv, stream=stream, split=split)
    context_kv_store(kv, positions, slots, cos_sin, caches, H, k_eps, stream=stream)
    return kv
