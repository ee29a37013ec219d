"""Chunk chain on one GPU: a long sequence processed as consecutive pipeline
chunks through their boundary states.

Source: Pith review of StateFlow, "What carries the argument": forward
chaining S_{i+1}^in = S_i^out (Eq. 5) and backward chaining
Sbar_i^out = Sbar_{i+1}^in (Eq. 7).  Chunks run in order, which is one legal
schedule of the page's partial order (Eq. 8) on a single device.  With B = 1
each chunk is a view into the sequence tensors, so no data is copied; every
chunk is one call of the C ABI.
"""
import math

import torch

from . import _lib


def split_lengths(lengths, f, multiple=64):
    """The page's split of a chunk at fraction f (Pith review of StateFlow,
    "Assumptions & free parameters", split fraction for overlap; Figure 2
    caption): every chunk of n tokens becomes two consecutive parts, the
    first of round(f n / multiple) * multiple tokens (whole kernel blocks) and
    the rest.  A chunk too short for two non-empty parts stays whole.  Run
    overlapped, part b's state-independent launches go beside part a's
    boundary-state chain and output, and the next chunk's part a beside part
    b's."""
    if not 0.0 < f < 1.0:
        raise ValueError("split fraction must be in (0, 1), got %r" % (f,))
    out = []
    for n in lengths:
        a = int(math.floor(f * n / multiple + 0.5)) * multiple
        out += [a, n - a] if 0 < a < n else [n]
    return out


def _bounds(lengths, T):
    if sum(lengths) != T or min(lengths) <= 0:
        raise ValueError("chunk lengths %r do not partition T=%d" % (lengths, T))
    b = [0]
    for n in lengths:
        b.append(b[-1] + n)
    return b


def _overlapped(n, begin, end, stream, side, order):
    """Split-and-overlap over chunks in ``order``: chunk i's BEGIN launches
    (independent of the boundary state) run on ``side`` while the previous
    chunk's END launches run on ``stream``.  Chunks alternate between two
    workspaces, so a BEGIN waits only for the END two chunks back, and every
    END waits for its own BEGIN (Pith review of StateFlow, Figure 2 caption).
    begin(i, slot) / end(i, slot) enqueue the launches on the given stream."""
    side.wait_stream(stream)
    ev_end = {}
    begin(order[0], 0)
    ev_begin = side.record_event()
    for n_i, i in enumerate(order):
        stream.wait_event(ev_begin)
        end(i, n_i % 2)
        ev_end[n_i] = stream.record_event()
        if n_i + 1 < n:
            if n_i >= 1:
                side.wait_event(ev_end[n_i - 1])  # the END that last used this workspace
            begin(order[n_i + 1], (n_i + 1) % 2)
            ev_begin = side.record_event()


def _ws_pair(workspaces, shapes, backward, dev, streams):
    if workspaces is not None:
        return workspaces
    need = max(_lib.workspace_bytes(s, backward=backward) for s in shapes)
    ws = [_lib.alloc_workspace(need, dev), _lib.alloc_workspace(need, dev)]
    _used_on(streams, *ws)
    return ws


def _used_on(streams, *tensors):
    """Buffers allocated here (on the current stream) that kernels on
    ``streams`` use: see _lib.used_on."""
    for st in streams:
        _lib.used_on(st, *tensors)


def chain_fwd(q, k, v, alpha, beta, S_in, lengths, o=None, seg_blocks=0, stream=None,
              save=False, overlap=False, side_stream=None, workspaces=None, saved=None,
              states=None, split=None):
    """Forward over consecutive chunks.  Returns (o, states) where states[i]
    is chunk i's entry state ([B,H,Dv,Dk] fp32; states[0] is S_in or zeros)
    and states[-1] the final state.  With ``save`` every chunk runs the saving
    forward and the return value is (o, states, saved), saved[i] being chunk
    i's buffer for the saved backward.

    ``split`` = f cuts every chunk into two parts at fraction f
    (split_lengths) and runs the parts as chunks: ``states`` and ``saved``
    then hold one entry per part (plus the final state), and chain_bwd takes
    the same ``split``.  Results equal the unsplit chain within rounding.

    ``overlap`` runs each chunk as its two launch groups, the next chunk's
    state-independent group on ``side_stream`` (a new default-priority stream
    when None) while the current chunk's chain and output run on ``stream``;
    results are bitwise those of the plain loop.  ``workspaces`` (two
    tensors), ``saved`` and ``states`` (len(lengths) + 1 tensors, states[0]
    the entry state) may be preallocated."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if B != 1:
        raise ValueError("chunk views need B == 1")
    if split is not None:
        lengths = split_lengths(lengths, split)
    bnd = _bounds(lengths, T)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
        _used_on([stream, side_stream], o)
    if overlap:
        dev = q.device
        main = stream if stream is not None else torch.cuda.current_stream(dev)
        side = side_stream if side_stream is not None else torch.cuda.Stream(device=dev)
        shapes = [_lib.make_shape(B, n, H, Dk, Dv, q.dtype, seg_blocks) for n in lengths]
        ws = _ws_pair(workspaces, shapes, False, dev, [main, side])
        if save and saved is None:
            saved = [_lib.alloc_workspace(_lib.saved_bytes(s), dev) for s in shapes]
            _used_on([main, side], *saved)
        if states is None:
            states = [S_in if S_in is not None else
                      torch.zeros((B, H, Dv, Dk), dtype=torch.float32, device=dev)]
            states += [torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
                       for _ in lengths]
            _used_on([main, side], *states[1:])
            if S_in is None:
                _used_on([main, side], states[0])
        sv = saved if save else [None] * len(lengths)

        def call(i, slot, st, phase):
            sl = slice(bnd[i], bnd[i + 1])
            _lib.chunk_fwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], states[i],
                           o=o[:, sl], S_out=states[i + 1], seg_blocks=seg_blocks,
                           workspace=ws[slot], stream=st, saved=sv[i], phase=phase)

        _overlapped(len(lengths), lambda i, slot: call(i, slot, side, _lib.PHASE_BEGIN),
                    lambda i, slot: call(i, slot, main, _lib.PHASE_END), main, side,
                    list(range(len(lengths))))
        return (o, states, saved) if save else (o, states)
    states = [S_in if S_in is not None else
              torch.zeros((B, H, Dv, Dk), dtype=torch.float32, device=q.device)]
    if S_in is None:
        _used_on([stream], states[0])
    saved = []
    for i in range(len(lengths)):
        sl = slice(bnd[i], bnd[i + 1])
        S_next = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
        _used_on([stream], S_next)
        r = _lib.chunk_fwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], states[i],
                           o=o[:, sl], S_out=S_next, seg_blocks=seg_blocks, stream=stream,
                           saved=True if save else None)
        if save:
            saved.append(r[2])
        states.append(S_next)
    return (o, states, saved) if save else (o, states)


def chain_bwd(q, k, v, alpha, beta, dO, dS_out, lengths, states, grads=None, seg_blocks=0,
              stream=None, saved=None, overlap=False, side_stream=None, workspaces=None,
              state_grads=None, split=None):
    """Backward over consecutive chunks, last chunk first, each chunk's
    entry-state gradient feeding the previous chunk's exit gradient.
    ``states`` are the entry states from chain_fwd; ``saved`` the per-chunk
    buffers of a saving chain_fwd (the recompute backward runs without them;
    ``states`` may then be None).  Returns (dq, dk, dv, dalpha, dbeta, dS_in).

    ``overlap`` (saved backward only) runs each chunk's state-independent
    launch group on ``side_stream`` while the later chunk's chain and
    gradients run on ``stream``, bitwise equal to the plain loop.
    ``state_grads`` may preallocate the len(lengths) entry-state gradients.
    ``split``: as in chain_fwd (the same f as the forward that produced
    ``states`` / ``saved``); chunks are then its parts."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if B != 1:
        raise ValueError("chunk views need B == 1")
    if split is not None:
        lengths = split_lengths(lengths, split)
    bnd = _bounds(lengths, T)
    if saved is not None and len(saved) != len(lengths):
        raise ValueError("%d saved buffers for %d chunks (was the forward split the same way?)"
                         % (len(saved), len(lengths)))
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(alpha), torch.empty_like(beta))
        _used_on([stream, side_stream], *grads)
    dq, dk, dv, da, db = grads
    if overlap:
        if saved is None:
            raise ValueError("the overlapped backward needs the saved buffers")
        dev = q.device
        main = stream if stream is not None else torch.cuda.current_stream(dev)
        side = side_stream if side_stream is not None else torch.cuda.Stream(device=dev)
        shapes = [_lib.make_shape(B, n, H, Dk, Dv, q.dtype, seg_blocks) for n in lengths]
        ws = _ws_pair(workspaces, shapes, True, dev, [main, side])
        if state_grads is None:
            state_grads = [torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
                           for _ in lengths]
            _used_on([main, side], *state_grads)
        n = len(lengths)

        def call(i, slot, st, phase):
            sl = slice(bnd[i], bnd[i + 1])
            G = dS_out if i == n - 1 else state_grads[i + 1]
            _lib.chunk_bwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], None,
                           dO[:, sl], G, grads=(dq[:, sl], dk[:, sl], dv[:, sl], da[:, sl],
                                                db[:, sl], state_grads[i]),
                           seg_blocks=seg_blocks, workspace=ws[slot], stream=st, saved=saved[i],
                           phase=phase)

        _overlapped(n, lambda i, slot: call(i, slot, side, _lib.PHASE_BEGIN),
                    lambda i, slot: call(i, slot, main, _lib.PHASE_END), main, side,
                    list(range(n - 1, -1, -1)))
        return dq, dk, dv, da, db, state_grads[0]
    G = dS_out
    for i in range(len(lengths) - 1, -1, -1):
        sl = slice(bnd[i], bnd[i + 1])
        G_prev = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
        _used_on([stream], G_prev)
        _lib.chunk_bwd(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl],
                       None if saved is not None else states[i],
                       dO[:, sl], G, grads=(dq[:, sl], dk[:, sl], dv[:, sl], da[:, sl],
                                            db[:, sl], G_prev),
                       seg_blocks=seg_blocks, stream=stream,
                       saved=None if saved is None else saved[i])
        G = G_prev
    return dq, dk, dv, da, db, G
