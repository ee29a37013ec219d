"""ctypes binding of libsf_gdn.so (the C ABI in include/sf_gdn.h).

Argument marshalling only: torch provides device memory and the stream, and
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or fails, calls raise.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsf_gdn.so")

SF_OK, SF_ERR_INVALID_ARG, SF_ERR_UNSUPPORTED, SF_ERR_WORKSPACE, SF_ERR_HIP = range(5)
SF_DTYPE_F32, SF_DTYPE_BF16 = 0, 1

_DTYPES = {torch.float32: SF_DTYPE_F32, torch.bfloat16: SF_DTYPE_BF16}

# Every function the header declares, with (restype, argtypes).
_vp, _cvp, _fp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_sz = ctypes.c_size_t


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("dtype", ctypes.c_int),
                ("seg_blocks", ctypes.c_int)]


class ConvShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("C", ctypes.c_int),
                ("W", ctypes.c_int), ("dtype", ctypes.c_int), ("act", ctypes.c_int)]


SIGNATURES = {
    "sf_gdn_chunk_fwd_workspace_size": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(_sz)]),
    "sf_gdn_chunk_bwd_workspace_size": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(_sz)]),
    "sf_gdn_chunk_fwd": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 8 + [_vp, _sz, _vp]),
    "sf_gdn_chunk_bwd": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 14 + [_vp, _sz, _vp]),
    "sf_gdn_chunk_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 8 + [_vp]),
    "sf_gdn_chunk_saved_size": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(_sz)]),
    "sf_gdn_segment_plan": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_int)]),
    "sf_gdn_chunk_fwd_save": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 9 + [_sz, _vp, _sz, _vp]),
    "sf_gdn_chunk_bwd_saved": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 6 + [_sz] + [_vp] * 8
                               + [_vp, _sz, _vp]),
    "sf_gdn_chunk_fwd_split": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 9
                               + [_sz, _vp, _sz, ctypes.c_int, _vp]),
    "sf_gdn_chunk_bwd_saved_split": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 6 + [_sz]
                                     + [_vp] * 8 + [_vp, _sz, ctypes.c_int, _vp]),
    "sf_gdn_shortconv_fwd": (ctypes.c_int, [ctypes.POINTER(ConvShape)] + [_vp] * 6),
    "sf_gdn_shortconv_bwd_workspace_size": (ctypes.c_int, [ctypes.POINTER(ConvShape),
                                                           ctypes.POINTER(_sz)]),
    "sf_gdn_shortconv_bwd": (ctypes.c_int, [ctypes.POINTER(ConvShape)] + [_vp] * 9 + [_sz, _vp]),
    "sf_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sf_last_error_message": (ctypes.c_char_p, []),
    "sf_gdn_version": (ctypes.c_char_p, []),
    "sf_gdn_profile_begin": (ctypes.c_int, [ctypes.c_int]),
    "sf_gdn_profile_end": (ctypes.c_int, []),
    "sf_gdn_profile_kernel_count": (ctypes.c_int, []),
    "sf_gdn_profile_kernel": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                             ctypes.POINTER(ctypes.c_longlong),
                                             ctypes.POINTER(ctypes.c_double)]),
}

_lib = None


# Launch groups of a chunk call (sf_gdn_chunk_fwd_split, sf_gdn_chunk_bwd_saved_split).
PHASE_ALL, PHASE_BEGIN, PHASE_END = 0, 1, 2


class GDNError(RuntimeError):
    def __init__(self, status, where, msg):
        super().__init__("%s: %s (%s)" % (where, msg, status_string(status)))
        self.status = status


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsf_gdn.so is not built; run "
                           "`python -m linear_recurrence_chunked_gated_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load().sf_status_string(int(status)).decode()


def _check(status, where):
    if status != SF_OK:
        raise GDNError(status, where, load().sf_last_error_message().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def used_on(stream, *tensors):
    """Mark tensors that this module allocated on the current stream as in
    use by ``stream`` when the kernels run there, so that the caching
    allocator does not hand their memory to current-stream work before the
    kernels are done (tensor.record_stream).  No-op for the current stream."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None and t.numel() > 0:
            t.record_stream(stream)


def make_shape(B, T, H, Dk, Dv, dtype, seg_blocks=0):
    if isinstance(dtype, torch.dtype):
        if dtype not in _DTYPES:
            raise TypeError("q/k/v must be bfloat16 or float32, got %s" % dtype)
        dtype = _DTYPES[dtype]
    return Shape(B, T, H, Dk, Dv, dtype, seg_blocks)


def workspace_bytes(shape, backward=False):
    n = ctypes.c_size_t(0)
    fn = load().sf_gdn_chunk_bwd_workspace_size if backward else load().sf_gdn_chunk_fwd_workspace_size
    _check(fn(ctypes.byref(shape), ctypes.byref(n)), "workspace_size")
    return n.value


def segment_plan(shape):
    """(blocks per segment, segments) of the in-chunk scan for `shape`."""
    L, P = ctypes.c_int(0), ctypes.c_int(0)
    _check(load().sf_gdn_segment_plan(ctypes.byref(shape), ctypes.byref(L), ctypes.byref(P)),
           "segment_plan")
    return L.value, P.value


def alloc_workspace(nbytes, device):
    """A 256-byte aligned uint8 view of at least nbytes (None when 0)."""
    if nbytes == 0:
        return None
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + nbytes]


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError("%s is required" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def saved_bytes(shape):
    n = ctypes.c_size_t(0)
    _check(load().sf_gdn_chunk_saved_size(ctypes.byref(shape), ctypes.byref(n)), "saved_size")
    return n.value


def chunk_fwd(q, k, v, alpha, beta, S_in=None, o=None, S_out=None, seg_blocks=0,
              workspace=None, stream=None, saved=None, phase=PHASE_ALL):
    """sf_gdn_chunk_fwd on torch tensors.  Returns (o, S_out).

    With ``saved`` (a uint8 tensor of at least ``saved_bytes`` bytes, 256-byte
    aligned, or True to allocate one) the saving forward runs and the return
    value is (o, S_out, saved).  ``phase`` selects one launch group
    (sf_gdn_chunk_fwd_split): PHASE_BEGIN then PHASE_END with the same
    arguments and workspace equals one PHASE_ALL call."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(q, "q", q.dtype, (B, T, H, Dk), dev)
    _need(k, "k", q.dtype, (B, T, H, Dk), dev)
    _need(v, "v", q.dtype, (B, T, H, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if S_in is not None:
        _need(S_in, "S_in", torch.float32, (B, H, Dv, Dk), dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
        used_on(stream, o)
    _need(o, "o", q.dtype, (B, T, H, Dv), dev)
    if S_out is None:
        S_out = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
        used_on(stream, S_out)
    _need(S_out, "S_out", torch.float32, (B, H, Dv, Dk), dev)
    shape = make_shape(B, T, H, Dk, Dv, q.dtype, seg_blocks)
    need = workspace_bytes(shape)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
        used_on(stream, workspace)
    wsn = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    if saved is True:
        n = saved_bytes(shape)
        saved = (alloc_workspace(n, dev) if n else
                 torch.empty(0, dtype=torch.uint8, device=dev))
        used_on(stream, saved)
    if phase != PHASE_ALL:
        st = load().sf_gdn_chunk_fwd_split(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(alpha), _ptr(beta), _ptr(S_in), _ptr(o),
                                           _ptr(S_out), _ptr(saved),
                                           ctypes.c_size_t(0 if saved is None else saved.numel()),
                                           _ptr(workspace), wsn, int(phase), _stream(stream))
        _check(st, "sf_gdn_chunk_fwd_split")
        return (o, S_out) if saved is None else (o, S_out, saved)
    if saved is None:
        st = load().sf_gdn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                     _ptr(beta), _ptr(S_in), _ptr(o), _ptr(S_out),
                                     _ptr(workspace), wsn, _stream(stream))
        _check(st, "sf_gdn_chunk_fwd")
        return o, S_out
    st = load().sf_gdn_chunk_fwd_save(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(beta), _ptr(S_in), _ptr(o), _ptr(S_out), _ptr(saved),
                                      ctypes.c_size_t(0 if saved is None else saved.numel()),
                                      _ptr(workspace), wsn, _stream(stream))
    _check(st, "sf_gdn_chunk_fwd_save")
    return o, S_out, saved


def chunk_fwd_noalloc(q, k, v, alpha, beta, S_in=None, o=None, S_out=None, seg_blocks=0,
                      stream=None):
    """sf_gdn_chunk_fwd_noalloc on torch tensors: the forward with the
    library's static workspace.  o and S_out must be preallocated by the
    caller when nothing may be allocated here.  Returns (o, S_out)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(q, "q", q.dtype, (B, T, H, Dk), dev)
    _need(k, "k", q.dtype, (B, T, H, Dk), dev)
    _need(v, "v", q.dtype, (B, T, H, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if S_in is not None:
        _need(S_in, "S_in", torch.float32, (B, H, Dv, Dk), dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
        used_on(stream, o)
    _need(o, "o", q.dtype, (B, T, H, Dv), dev)
    if S_out is None:
        S_out = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
        used_on(stream, S_out)
    _need(S_out, "S_out", torch.float32, (B, H, Dv, Dk), dev)
    shape = make_shape(B, T, H, Dk, Dv, q.dtype, seg_blocks)
    st = load().sf_gdn_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(alpha), _ptr(beta), _ptr(S_in), _ptr(o),
                                         _ptr(S_out), _stream(stream))
    _check(st, "sf_gdn_chunk_fwd_noalloc")
    return o, S_out


def chunk_bwd(q, k, v, alpha, beta, S_in, dO, dS_out=None, grads=None, seg_blocks=0,
              workspace=None, stream=None, saved=None, phase=PHASE_ALL):
    """sf_gdn_chunk_bwd on torch tensors (sf_gdn_chunk_bwd_saved when
    ``saved`` holds the buffer of a saving forward; S_in is then unused).
    ``phase`` selects one launch group of the saved backward
    (sf_gdn_chunk_bwd_saved_split).

    Returns (dq, dk, dv, dalpha, dbeta, dS_in).  ``grads`` may supply
    preallocated outputs in that order (dS_in may be None there)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t, n, dt, shp in ((q, "q", q.dtype, (B, T, H, Dk)), (k, "k", q.dtype, (B, T, H, Dk)),
                          (v, "v", q.dtype, (B, T, H, Dv)), (dO, "dO", q.dtype, (B, T, H, Dv)),
                          (alpha, "alpha", torch.float32, (B, T, H)),
                          (beta, "beta", torch.float32, (B, T, H))):
        _need(t, n, dt, shp, dev)
    if S_in is not None and saved is None:
        _need(S_in, "S_in", torch.float32, (B, H, Dv, Dk), dev)
    if dS_out is not None:
        _need(dS_out, "dS_out", torch.float32, (B, H, Dv, Dk), dev)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(alpha), torch.empty_like(beta),
                 torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev))
        used_on(stream, *grads)
    dq, dk, dv, da, db, dS_in = grads
    shape = make_shape(B, T, H, Dk, Dv, q.dtype, seg_blocks)
    need = workspace_bytes(shape, backward=True)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
        used_on(stream, workspace)
    wsn = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    if phase != PHASE_ALL:
        if saved is None:
            raise ValueError("the split backward needs the saved buffer of a saving forward")
        st = load().sf_gdn_chunk_bwd_saved_split(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(saved),
            ctypes.c_size_t(saved.numel()), _ptr(dO), _ptr(dS_out), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(da), _ptr(db), _ptr(dS_in), _ptr(workspace), wsn, int(phase), _stream(stream))
        _check(st, "sf_gdn_chunk_bwd_saved_split")
    elif saved is None:
        st = load().sf_gdn_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                     _ptr(beta), _ptr(S_in), _ptr(dO), _ptr(dS_out), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(dS_in),
                                     _ptr(workspace), wsn, _stream(stream))
        _check(st, "sf_gdn_chunk_bwd")
    else:
        st = load().sf_gdn_chunk_bwd_saved(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(alpha), _ptr(beta), _ptr(saved),
                                           ctypes.c_size_t(saved.numel()), _ptr(dO), _ptr(dS_out),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(db),
                                           _ptr(dS_in), _ptr(workspace), wsn, _stream(stream))
        _check(st, "sf_gdn_chunk_bwd_saved")
    return dq, dk, dv, da, db, dS_in


def conv_shape(B, T, C, W, dtype, act=0):
    if isinstance(dtype, torch.dtype):
        if dtype not in _DTYPES:
            raise TypeError("x must be bfloat16 or float32, got %s" % dtype)
        dtype = _DTYPES[dtype]
    return ConvShape(B, T, C, W, dtype, int(act))


def shortconv_bwd_workspace_bytes(shape):
    n = ctypes.c_size_t(0)
    _check(load().sf_gdn_shortconv_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "shortconv_bwd_workspace_size")
    return n.value


def shortconv_fwd(x, w, conv_in=None, act=0, y=None, conv_out=None, want_state=True,
                  stream=None):
    """sf_gdn_shortconv_fwd on torch tensors: x [B,T,C], w [C,W] fp32,
    conv_in [B,W-1,C] or None.  Returns (y, conv_out); conv_out is None when
    want_state is False."""
    B, T, C = x.shape
    W = w.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", x.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C, W), dev)
    if conv_in is not None:
        _need(conv_in, "conv_in", x.dtype, (B, W - 1, C), dev)
    if y is None:
        y = torch.empty_like(x)
        used_on(stream, y)
    _need(y, "y", x.dtype, (B, T, C), dev)
    if want_state and conv_out is None and W > 1:
        conv_out = torch.empty((B, W - 1, C), dtype=x.dtype, device=dev)
        used_on(stream, conv_out)
    shape = conv_shape(B, T, C, W, x.dtype, act)
    _check(load().sf_gdn_shortconv_fwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(conv_in),
                                       _ptr(y), _ptr(conv_out) if W > 1 else None,
                                       _stream(stream)), "sf_gdn_shortconv_fwd")
    return y, conv_out


def shortconv_bwd(x, w, conv_in, dy, dconv_out=None, act=0, dx=None, dw=None, want_state=True,
                  workspace=None, stream=None):
    """sf_gdn_shortconv_bwd on torch tensors.  Returns (dx, dw, dconv_in)."""
    B, T, C = x.shape
    W = w.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", x.dtype, (B, T, C), dev)
    _need(dy, "dy", x.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C, W), dev)
    for t, n in ((conv_in, "conv_in"), (dconv_out, "dconv_out")):
        if t is not None:
            _need(t, n, x.dtype, (B, W - 1, C), dev)
    if dx is None:
        dx = torch.empty_like(x)
        used_on(stream, dx)
    if dw is None:
        dw = torch.empty_like(w)
        used_on(stream, dw)
    dci = (torch.empty((B, W - 1, C), dtype=x.dtype, device=dev)
           if want_state and W > 1 else None)
    used_on(stream, dci)
    shape = conv_shape(B, T, C, W, x.dtype, act)
    need = shortconv_bwd_workspace_bytes(shape)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
        used_on(stream, workspace)
    _check(load().sf_gdn_shortconv_bwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(conv_in),
                                       _ptr(dy), _ptr(dconv_out), _ptr(dx), _ptr(dw), _ptr(dci),
                                       _ptr(workspace),
                                       ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                       _stream(stream)), "sf_gdn_shortconv_bwd")
    return dx, dw, dci


class profile:
    """Context manager: per-kernel HIP-event timing of the library's launches.

    After exit, ``.results`` maps kernel name -> (launches, total_ms)."""

    def __init__(self, capacity=65536):
        self.capacity = capacity
        self.results = {}

    def __enter__(self):
        _check(load().sf_gdn_profile_begin(int(self.capacity)), "sf_gdn_profile_begin")
        return self

    def __exit__(self, *exc):
        lib = load()
        _check(lib.sf_gdn_profile_end(), "sf_gdn_profile_end")
        for i in range(lib.sf_gdn_profile_kernel_count()):
            name = ctypes.c_char_p()
            n = ctypes.c_longlong()
            ms = ctypes.c_double()
            _check(lib.sf_gdn_profile_kernel(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
                   "sf_gdn_profile_kernel")
            self.results[name.value.decode()] = (n.value, ms.value)
        return False
