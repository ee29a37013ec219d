"""torch autograd over one chunk.

    gated_delta_chunk(q, k, v, alpha, beta, S_in=None, seg_blocks=0) -> (o, S_out)
    short_conv(x, w, conv_in=None, act=0)                           -> (y, conv_out)

The forward is the saving forward (sf_gdn_chunk_fwd_save: o and S_out, with
each block's entry state and V^new kept for the backward), and the backward is
sf_gdn_chunk_bwd_saved on the gradients autograd hands back for o and S_out
(zeros where an output took no part in the loss).  The gradient of S_in is the
chunk's boundary-state gradient dS_in ([SF] "What carries the argument",
Eq. 7), so chunks chained through S_in = previous S_out differentiate as one
sequence.  short_conv is the causal depthwise convolution ahead of the
recurrence (sf_gdn_shortconv_fwd / _bwd), whose W-1-token boundary state
chains the same way.  Argument marshalling only: both passes are the library's
kernels, and CPU tensors are refused as in chunk_fwd.
"""
import torch

from . import _lib


class _GatedDeltaChunk(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, alpha, beta, S_in, seg_blocks):
        o, S_out, saved = _lib.chunk_fwd(q, k, v, alpha, beta, S_in, seg_blocks=seg_blocks,
                                         saved=True)
        ctx.save_for_backward(q, k, v, alpha, beta)
        ctx.saved_states = saved  # the backward's per-block states; kept for the graph's life
        ctx.seg_blocks = seg_blocks
        ctx.has_s_in = S_in is not None
        return o, S_out

    @staticmethod
    def backward(ctx, dO, dS_out):
        q, k, v, alpha, beta = ctx.saved_tensors
        dq, dk, dv, dalpha, dbeta, dS_in = _lib.chunk_bwd(
            q, k, v, alpha, beta, None, dO.contiguous(), dS_out.contiguous(),
            seg_blocks=ctx.seg_blocks, saved=ctx.saved_states)
        return dq, dk, dv, dalpha, dbeta, (dS_in if ctx.has_s_in else None), None


def gated_delta_chunk(q, k, v, alpha, beta, S_in=None, seg_blocks=0):
    """(o, S_out) of one chunk, differentiable in q, k, v, alpha, beta and
    S_in.  Shapes and dtypes as chunk_fwd: q, k [B, T, H, Dk] and v [B, T, H,
    Dv] in bf16 or fp32 (contiguous), alpha, beta [B, T, H] fp32, S_in
    [B, H, Dv, Dk] fp32 or None (a zero state, which then gets no gradient)."""
    return _GatedDeltaChunk.apply(q, k, v, alpha, beta, S_in, seg_blocks)


class _ShortConv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, conv_in, act):
        y, conv_out = _lib.shortconv_fwd(x, w, conv_in, act=act)
        if conv_out is None:  # W = 1: no boundary state
            conv_out = x.new_zeros((x.shape[0], 0, x.shape[2]))
        ctx.save_for_backward(x, w, conv_in)
        ctx.act = act
        ctx.has_state = conv_in is not None
        return y, conv_out

    @staticmethod
    def backward(ctx, dy, dconv_out):
        x, w, conv_in = ctx.saved_tensors
        dstate = dconv_out.contiguous() if dconv_out.shape[1] > 0 else None
        dx, dw, dconv_in = _lib.shortconv_bwd(x, w, conv_in, dy.contiguous(), dstate, act=ctx.act,
                                              want_state=ctx.has_state)
        return dx, dw, (dconv_in if ctx.has_state else None), None


def short_conv(x, w, conv_in=None, act=0):
    """(y, conv_out) of the causal depthwise convolution over one chunk,
    differentiable in x, w and conv_in: x [B, T, C] bf16 or fp32, w [C, W]
    fp32, conv_in [B, W-1, C] in x's dtype or None (zeros, no gradient); act 0
    for none, 1 for SiLU."""
    return _ShortConv.apply(x, w, conv_in, act)
