"""torch autograd over one chunk.

    gated_delta_chunk(q, k, v, alpha, beta, S_in=None, seg_blocks=0) -> (o, S_out)

The forward is the saving forward (sf_gdn_chunk_fwd_save: o and S_out, with
each block's entry state and V^new kept for the backward), and the backward is
sf_gdn_chunk_bwd_saved on the gradients autograd hands back for o and S_out
(zeros where an output took no part in the loss).  The gradient of S_in is the
chunk's boundary-state gradient dS_in ([SF] "What carries the argument",
Eq. 7), so chunks chained through S_in = previous S_out differentiate as one
sequence.  Argument marshalling only: both passes are the library's kernels,
and CPU tensors are refused as in chunk_fwd.
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
