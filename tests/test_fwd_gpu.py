"""Forward parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance: max relative error (max |x - ref| / max |ref|, per head) <= 2e-2
for bf16 inputs and <= 1e-4 for fp32 inputs.  The oracle consumes exactly the
rounded values the device sees.
"""
import numpy as np
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
from gdn_testutil import TOL, assert_close, inputs, to_dev, oracle_args, head_slice, f64

pytestmark = pytest.mark.gpu


def run_fwd(d, seg_blocks=0):
    dd = to_dev(d)
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                         seg_blocks=seg_blocks)
    torch.cuda.synchronize()
    return f64(o), f64(S)


@pytest.mark.parametrize("B,T,H,D,dtype,s_in,decay,seg", [
    (1, 256, 2, 64, "f32", None, 1.0, 0),      # the fp32 shape, unchained
    (1, 256, 2, 64, "f32", 0.1, 0.01, 1),      # slow decay, one block per segment
    (2, 333, 3, 64, "f32", 0.1, 0.01, 2),      # ragged tail, B = 2
    (1, 256, 2, 128, "f32", None, 1.0, 0),     # fp32 at d = 128
    (2, 333, 2, 128, "f32", 0.1, 0.01, 2),     # fp32 at d = 128: ragged tail, B = 2
    (1, 1000, 2, 128, "f32", 0.1, 0.01, 3),    # fp32 at d = 128: ragged segments
    (1, 1000, 3, 128, "bf16", 0.1, 0.01, 0),   # ragged, several segments
    (2, 640, 2, 128, "bf16", None, 1.0, 3),
    (1, 1, 2, 128, "bf16", 0.1, 1.0, 0),       # single token
    (1, 63, 2, 64, "bf16", 0.1, 0.01, 0),      # one partial block
    (1, 65, 1, 128, "bf16", 0.1, 0.01, 1),     # one full block and one token
    (1, 2048, 4, 128, "bf16", 0.1, 0.01, 5),   # ragged segments (32 blocks / 5)
    (1, 1000, 2, 64, "bf16", 0.1, 0.01, 5),    # d = 64: segments of 5, 5, 5, 1 blocks
])
def test_fwd_matches_oracle(oracle_mod, B, T, H, D, dtype, s_in, decay, seg):
    d = inputs(B, T, H, D, dtype, seed=1000 + T + H, s_in_std=s_in, decay=decay)
    o, S = run_fwd(d, seg)
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    tol = TOL[dtype]
    assert_close("o", o, o_ref, tol, head_axis=2)
    assert_close("S_out", S, S_ref, tol, head_axis=1)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("decay", [1.0, 0.01])
def test_fp32_chained_4x64(oracle_mod, decay, D):
    """Four chunks of 64 tokens chained through S_in/S_out (Eq. 5) against
    the unchunked oracle, fp32 bar."""
    d = inputs(1, 256, 2, D, "f32", seed=20260000, decay=decay)
    dd = to_dev(d)
    o, states = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None, [64] * 4)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["f32"], head_axis=2)
    assert_close("S_out", f64(states[-1]), S_ref, TOL["f32"], head_axis=1)


@pytest.mark.parametrize("decay", [1.0, 0.01])
def test_bf16_chained_8x1024(oracle_mod, decay):
    """H=16, T=8192, d=128, eight chunks of 1024 chained, against the
    unchunked oracle."""
    d = inputs(1, 8192, 16, 128, "bf16", seed=20260001, decay=decay)
    dd = to_dev(d)
    o, states = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None, [1024] * 8)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(states[-1]), S_ref, TOL["bf16"], head_axis=1)


def test_chunked_equals_unchunked_within_tolerance():
    d = to_dev(inputs(1, 4096, 4, 128, "bf16", seed=7, s_in_std=0.1, decay=0.01))
    o1, S1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    lengths = [960, 64, 1984, 1088]
    o2, st = gdn.chain_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"], lengths)
    torch.cuda.synchronize()
    assert_close("o", f64(o2), f64(o1), TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(st[-1]), f64(S1), TOL["bf16"], head_axis=1)


def test_bitwise_when_segments_align():
    """With one block per segment, a chunk boundary at a block boundary gives
    the same operations in the same order: chained == unchained bit for bit."""
    d = to_dev(inputs(1, 1024, 2, 128, "bf16", seed=8, s_in_std=0.1, decay=0.01))
    o1, S1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"], seg_blocks=1)
    o2, st = gdn.chain_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"], [512, 512],
                           seg_blocks=1)
    torch.cuda.synchronize()
    # The chain inside one call composes segment maps, so only the outputs of
    # the first chunk are guaranteed identical; compare within tolerance for
    # the rest and bitwise for chunk 0.
    assert torch.equal(o1[:, :512], o2[:, :512])
    assert_close("o", f64(o2), f64(o1), TOL["bf16"], head_axis=2)


def test_deterministic():
    d = to_dev(inputs(1, 3000, 3, 128, "bf16", seed=9, s_in_std=0.1))
    r1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    r2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_empty_chunk_passes_state():
    d = to_dev(inputs(1, 0, 2, 64, "bf16", seed=10, s_in_std=0.1))
    o, S = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 64)
    assert torch.equal(S, d["S_in"])


def test_full_size_h32_t65536_sampled_heads(oracle_mod):
    """One GPU's share of a 256K-token sequence (T=65536, H=32, d=128, bf16,
    S_in ~ N(0, 0.1)), in the launch configuration the benchmark uses; the
    oracle checks four whole heads."""
    d = inputs(1, 65536, 32, 128, "bf16", seed=20260002, s_in_std=0.1)
    o, S = run_fwd(d)
    hs = [0, 11, 20, 31]
    sub = head_slice(d, hs)
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(sub))
    assert_close("o", o[:, :, hs], o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", S[:, hs], S_ref, TOL["bf16"], head_axis=1)


def test_full_size_h16_t65536_sampled_heads(oracle_mod):
    """The forward-only target shape (T=65536, H=16, d=128, bf16, S_in ~
    N(0, 0.1)), drawn on the device by the seeded generator as the benchmark
    draws it, in the launch configuration the benchmark times (16 segments
    of 64 blocks); the oracle checks four whole heads."""
    dd = inputs(1, 65536, 16, 128, "bf16", seed=20260102, s_in_std=0.1, device="cuda")
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
    torch.cuda.synchronize()
    hs = [2, 6, 9, 13]
    sub = head_slice(dd, hs)
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(sub))
    assert_close("o", f64(o[:, :, hs]), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(S[:, hs]), S_ref, TOL["bf16"], head_axis=1)


def test_nonuniform_chunk_lengths_are_block_multiples():
    lengths = chunk_lengths(262144, 8, 0.5)
    assert sum(lengths) == 262144 and all(n % 64 == 0 for n in lengths)
