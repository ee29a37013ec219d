"""ctypes wrapper of the fp64 token-loop oracle (TEST INFRASTRUCTURE).

Every array is upcast to C-contiguous float64 before the call, so callers can
pass the exact bf16- or fp32-rounded values the device sees.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def lib_path():
    return _LIB


def build(force=True):
    """Compile the oracle with gcc -O2 (no fast-math) and OpenMP."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_gdn_fwd.restype = i
    lib.oracle_gdn_fwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gdn_bwd.restype = i
    lib.oracle_gdn_bwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp,
                                   dp, dp, dp, dp, dp, dp, i]
    lib.oracle_shortconv_fwd.restype = None
    lib.oracle_shortconv_fwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp]
    lib.oracle_shortconv_bwd.restype = None
    lib.oracle_shortconv_bwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp]
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shape(q, v):
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    return B, T, H, Dk, Dv


def gdn_fwd(q, k, v, alpha, beta, S_in=None, nthreads=0, return_threads=False):
    """Token-by-token forward.  Returns (o, S_out) as float64 arrays.

    q, k: [B,T,H,Dk]; v: [B,T,H,Dv]; alpha, beta: [B,T,H];
    S_in: [B,H,Dv,Dk] or None (zeros).
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    S_in = None if S_in is None else _f64(S_in)
    B, T, H, Dk, Dv = _shape(q, v)
    o = np.zeros((B, T, H, Dv), np.float64)
    S_out = np.zeros((B, H, Dv, Dk), np.float64)
    nt = _load().oracle_gdn_fwd(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(S_in), _ptr(o), _ptr(S_out), int(nthreads))
    if nt < 0:
        raise RuntimeError("oracle_gdn_fwd failed (%d)" % nt)
    return (o, S_out, nt) if return_threads else (o, S_out)


def gdn_bwd(q, k, v, alpha, beta, S_in, dO, dS_out, nthreads=0, return_threads=False):
    """Analytic backward of L = <dO, o> + <dS_out, S_out>.

    Returns (dq, dk, dv, dalpha, dbeta, dS_in) as float64 arrays.  S_in and
    dS_out may be None (zeros).
    """
    q, k, v, alpha, beta, dO = map(_f64, (q, k, v, alpha, beta, dO))
    S_in = None if S_in is None else _f64(S_in)
    dS_out = None if dS_out is None else _f64(dS_out)
    B, T, H, Dk, Dv = _shape(q, v)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    da = np.zeros_like(alpha)
    db = np.zeros_like(beta)
    dS_in = np.zeros((B, H, Dv, Dk), np.float64)
    nt = _load().oracle_gdn_bwd(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(S_in), _ptr(dO), _ptr(dS_out), _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(dS_in),
                                int(nthreads))
    if nt < 0:
        raise RuntimeError("oracle_gdn_bwd failed (%d)" % nt)
    out = (dq, dk, dv, da, db, dS_in)
    return out + (nt,) if return_threads else out


def gdn_fwd_chained(q, k, v, alpha, beta, S_in, lengths, nthreads=0):
    """Forward over consecutive chunks of the given token lengths, passing
    each chunk's exit state on as the next chunk's entry state (Eq. 5).
    Returns (o, S_out, states) where states[i] is the entry state of chunk i
    and states[-1] the final state."""
    B, T, H, Dk, Dv = _shape(np.asarray(q), np.asarray(v))
    assert sum(lengths) == T
    o = np.zeros((B, T, H, Dv), np.float64)
    S = None if S_in is None else _f64(S_in)
    states = [np.zeros((B, H, Dv, Dk)) if S is None else S.copy()]
    t0 = 0
    for n in lengths:
        sl = slice(t0, t0 + n)
        oc, S = gdn_fwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], S,
                        nthreads=nthreads)
        o[:, sl] = oc
        states.append(S.copy())
        t0 += n
    return o, S, states


def gdn_bwd_chained(q, k, v, alpha, beta, S_in, dO, dS_out, lengths, nthreads=0):
    """Backward over consecutive chunks, last chunk first, passing each
    chunk's entry-state gradient on as the previous chunk's exit-state
    gradient (Eq. 7).  Entry states come from the chained forward."""
    q, k, v, alpha, beta, dO = map(_f64, (q, k, v, alpha, beta, dO))
    _, _, states = gdn_fwd_chained(q, k, v, alpha, beta, S_in, lengths, nthreads)
    B, T, H, Dk, Dv = _shape(q, v)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    da = np.zeros_like(alpha)
    db = np.zeros_like(beta)
    G = None if dS_out is None else _f64(dS_out)
    starts = np.concatenate([[0], np.cumsum(lengths)]).astype(int)
    for i in range(len(lengths) - 1, -1, -1):
        sl = slice(starts[i], starts[i + 1])
        r = gdn_bwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], states[i],
                    dO[:, sl], G, nthreads=nthreads)
        dq[:, sl], dk[:, sl], dv[:, sl], da[:, sl], db[:, sl] = r[:5]
        G = r[5]
    return dq, dk, dv, da, db, G


def shortconv_fwd(x, w, conv_in=None, act=0):
    """Causal depthwise convolution of one chunk with its boundary state.
    x: [B,T,C]; w: [C,W]; conv_in: [B,W-1,C] or None (zeros).
    Returns (y [B,T,C], conv_out [B,W-1,C]) as float64."""
    x, w = _f64(x), _f64(w)
    cin = None if conv_in is None else _f64(conv_in)
    B, T, C = x.shape
    W = w.shape[1]
    y = np.zeros((B, T, C), np.float64)
    cout = np.zeros((B, W - 1, C), np.float64)
    _load().oracle_shortconv_fwd(B, T, C, W, int(act), _ptr(x), _ptr(w), _ptr(cin), _ptr(y),
                                 _ptr(cout))
    return y, cout


def shortconv_bwd(x, w, conv_in, dy, dconv_out=None, act=0):
    """Gradients of <dy, y> + <dconv_out, conv_out>: (dx, dw, dconv_in)."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    cin = None if conv_in is None else _f64(conv_in)
    dco = None if dconv_out is None else _f64(dconv_out)
    B, T, C = x.shape
    W = w.shape[1]
    dx = np.zeros((B, T, C), np.float64)
    dw = np.zeros((C, W), np.float64)
    dcin = np.zeros((B, W - 1, C), np.float64)
    _load().oracle_shortconv_bwd(B, T, C, W, int(act), _ptr(x), _ptr(w), _ptr(cin), _ptr(dy),
                                 _ptr(dco), _ptr(dx), _ptr(dw), _ptr(dcin))
    return dx, dw, dcin
