"""Parity at the ends of the gates' range, and fp32 through a long segment
chain: the HIP forward and backward through the C ABI against the fp64 oracle
with

  strong  alpha = exp(-10 softplus(z)), down to about 1e-13: the decay inside
          one 64-token block spans hundreds of e-folds, so Gamma and gamma
          underflow to zero within the block;
  none    alpha = 1 exactly (no decay: the plain delta rule);
  beta0   beta = 0 (no writes: pure decay, T = I, A = 0), with slow decay so
          that the carried state stays within fp32 range;
  beta1   alpha = beta = 1 (each token overwrites the state along k_t).

The recurrence is defined for 0 < alpha <= 1 and 0 <= beta <= 1; these are the
degenerate points of that range.  Same tolerances as the other parity tests
(per head: bf16 2e-2, fp32 1e-4), ragged T and several segments per head.

The gate gradient is checked both as dalpha and as alpha * dalpha, the
gradient with respect to log alpha.  With strong decay a token's alpha can be
1e-13 while its dalpha is of the head's scale: d log alpha is then of alpha's
order, and dalpha = d log alpha / alpha is only accurate if every term of
d log alpha is formed with alpha as a factor rather than as a difference of
terms of the block's scale.
"""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from gdn_testutil import TOL, assert_close, inputs, to_dev, oracle_args, f64, as_f64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS_in")
HEAD_AXIS = (2, 2, 2, 2, 2, 1)


def gated_inputs(mode, B, T, H, D, dtype, seed):
    decay = {"strong": 10.0, "none": 0.0, "beta0": 0.01}.get(mode, 1.0)
    d = inputs(B, T, H, D, dtype, seed=seed, s_in_std=0.1, grads=True, decay=decay)
    if mode == "beta0":
        d["beta"] = torch.zeros_like(d["beta"])
    elif mode == "beta1":
        d["alpha"] = torch.ones_like(d["alpha"])
        d["beta"] = torch.ones_like(d["beta"])
    return d


CASES = [
    (mode, B, T, H, D, dtype, seg)
    for mode in ("strong", "none", "beta0", "beta1")
    for (B, T, H, D, dtype, seg) in ((1, 1000, 2, 128, "bf16", 3), (2, 333, 2, 64, "f32", 2))
] + [
    # strong decay on the other two kernel forms: four waves per workgroup
    # (d = 64), and the gradient kernel with its tiles in global memory (fp32
    # at d = 128)
    ("strong", 1, 700, 2, 64, "bf16", 2),
    ("strong", 1, 333, 2, 128, "f32", 2),
]


@pytest.mark.parametrize("mode,B,T,H,D,dtype,seg", CASES)
def test_gate_extremes_fwd_bwd(oracle_mod, mode, B, T, H, D, dtype, seg):
    d = gated_inputs(mode, B, T, H, D, dtype, seed=9500 + T + D)
    dd = to_dev(d)
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                         seg_blocks=seg)
    grads = gdn.chunk_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                          dd["dO"], dd["dS_out"], seg_blocks=seg)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, tol, head_axis=2)
    assert_close("S_out", f64(S), S_ref, tol, head_axis=1)
    ref = oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))
    alpha = as_f64(d["alpha"])
    assert_close("alpha * dalpha", alpha * f64(grads[3]), alpha * ref[3], tol, head_axis=2)
    for name, g, r, ax in zip(NAMES, grads, ref, HEAD_AXIS):
        assert_close(name, f64(g), r, tol, head_axis=ax)


@pytest.mark.parametrize("D,decay", [(64, 0.0), (128, 0.0), (128, 0.01)])
def test_fp32_long_chain(oracle_mod, D, decay):
    """fp32 within 1e-4 through 128 segments of one block each (127 steps of
    the in-chunk segment chain, whose products run on split bf16 operands),
    with no decay, so nothing of an early segment's state fades before the
    chunk's end, and with slow decay."""
    d = inputs(1, 8192, 2, D, "f32", seed=9900 + D, s_in_std=0.1, grads=True, decay=decay)
    dd = to_dev(d)
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                         seg_blocks=1)
    grads = gdn.chunk_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                          dd["dO"], dd["dS_out"], seg_blocks=1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["f32"], head_axis=2)
    assert_close("S_out", f64(S), S_ref, TOL["f32"], head_axis=1)
    ref = oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))
    for name, g, r, ax in zip(NAMES, grads, ref, HEAD_AXIS):
        assert_close(name, f64(g), r, TOL["f32"], head_axis=ax)
