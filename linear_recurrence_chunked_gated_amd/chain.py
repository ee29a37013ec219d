"""Chunk chain on one GPU: a long sequence processed as consecutive pipeline
chunks through their boundary states.

Source: Pith review of StateFlow, "What carries the argument": forward
chaining S_{i+1}^in = S_i^out (Eq. 5) and backward chaining
Sbar_i^out = Sbar_{i+1}^in (Eq. 7).  Chunks run in order, which is one legal
schedule of the page's partial order (Eq. 8) on a single device.  With B = 1
each chunk is a view into the sequence tensors, so no data is copied; every
chunk is one call of the C ABI.
"""
import torch

from . import _lib


def _bounds(lengths, T):
    if sum(lengths) != T or min(lengths) <= 0:
        raise ValueError("chunk lengths %r do not partition T=%d" % (lengths, T))
    b = [0]
    for n in lengths:
        b.append(b[-1] + n)
    return b


def chain_fwd(q, k, v, alpha, beta, S_in, lengths, o=None, seg_blocks=0, stream=None,
              save=False):
    """Forward over consecutive chunks.  Returns (o, states) where states[i]
    is chunk i's entry state ([B,H,Dv,Dk] fp32; states[0] is S_in or zeros)
    and states[-1] the final state.  With ``save`` every chunk runs the saving
    forward and the return value is (o, states, saved), saved[i] being chunk
    i's buffer for the saved backward."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if B != 1:
        raise ValueError("chunk views need B == 1")
    bnd = _bounds(lengths, T)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    states = [S_in if S_in is not None else
              torch.zeros((B, H, Dv, Dk), dtype=torch.float32, device=q.device)]
    saved = []
    for i in range(len(lengths)):
        sl = slice(bnd[i], bnd[i + 1])
        S_next = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
        r = _lib.chunk_fwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], states[i],
                           o=o[:, sl], S_out=S_next, seg_blocks=seg_blocks, stream=stream,
                           saved=True if save else None)
        if save:
            saved.append(r[2])
        states.append(S_next)
    return (o, states, saved) if save else (o, states)


def chain_bwd(q, k, v, alpha, beta, dO, dS_out, lengths, states, grads=None, seg_blocks=0,
              stream=None, saved=None):
    """Backward over consecutive chunks, last chunk first, each chunk's
    entry-state gradient feeding the previous chunk's exit gradient.
    ``states`` are the entry states from chain_fwd; ``saved`` the per-chunk
    buffers of a saving chain_fwd (the recompute backward runs without them;
    ``states`` may then be None).  Returns (dq, dk, dv, dalpha, dbeta, dS_in)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if B != 1:
        raise ValueError("chunk views need B == 1")
    bnd = _bounds(lengths, T)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(alpha), torch.empty_like(beta))
    dq, dk, dv, da, db = grads
    G = dS_out
    for i in range(len(lengths) - 1, -1, -1):
        sl = slice(bnd[i], bnd[i + 1])
        G_prev = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
        _lib.chunk_bwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl],
                       None if saved is not None else states[i],
                       dO[:, sl], G, grads=(dq[:, sl], dk[:, sl], dv[:, sl], da[:, sl],
                                            db[:, sl], G_prev),
                       seg_blocks=seg_blocks, stream=stream,
                       saved=None if saved is None else saved[i])
        G = G_prev
    return dq, dk, dv, da, db, G
