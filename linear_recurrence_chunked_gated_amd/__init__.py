"""MI355X (gfx950) HIP implementation of one pipeline chunk of the gated
delta-rule recurrence (Gated DeltaNet), forward and backward, behind the C ABI
in include/sf_gdn.h.

    chunk_fwd(q, k, v, alpha, beta, S_in)            -> (o, S_out)
    chunk_bwd(q, k, v, alpha, beta, S_in, dO, dS_out)
                                 -> (dq, dk, dv, dalpha, dbeta, dS_in)
    chain_fwd / chain_bwd: consecutive chunks through their boundary states.
    gated_delta_chunk(q, k, v, alpha, beta, S_in)    -> (o, S_out), torch autograd
    short_conv(x, w, conv_in)                        -> (y, conv_out), torch autograd
    shortconv_fwd(x, w, conv_in)                     -> (y, conv_out)
    shortconv_bwd(x, w, conv_in, dy, dconv_out)      -> (dx, dw, dconv_in)

Imports are lazy so that the input generator and the planner load without the
HIP library.
"""
__all__ = ["chunk_fwd", "chunk_bwd", "chain_fwd", "chain_bwd", "gated_delta_chunk", "short_conv",
           "shortconv_fwd", "shortconv_bwd", "profile", "GDNError"]


def __getattr__(name):
    if name in ("chunk_fwd", "chunk_bwd", "shortconv_fwd", "shortconv_bwd", "profile", "GDNError"):
        from . import _lib
        return getattr(_lib, name)
    if name in ("chain_fwd", "chain_bwd"):
        from . import chain
        return getattr(chain, name)
    if name in ("gated_delta_chunk", "short_conv"):
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(name)
