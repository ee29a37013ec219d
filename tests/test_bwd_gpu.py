"""Backward parity: the HIP chunk backward through the C ABI against the fp64
oracle's analytic backward, plus a finite-difference probe of the loss
L = <dO, o> + <dS_out, S_out> evaluated by the oracle.

Tolerance: max relative error per tensor (per head) <= 2e-2 for bf16 inputs,
<= 1e-4 for fp32 inputs.
"""
import numpy as np
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
from gdn_testutil import TOL, assert_close, inputs, to_dev, oracle_args, head_slice, f64, as_f64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS_in")
HEAD_AXIS = (2, 2, 2, 2, 2, 1)


def run_bwd(d, seg_blocks=0):
    dd = to_dev(d)
    r = gdn.chunk_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"], dd["dO"],
                      dd["dS_out"], seg_blocks=seg_blocks)
    torch.cuda.synchronize()
    return [f64(x) for x in r]


def oracle_bwd(oracle_mod, d):
    return oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))


def check_all(got, ref, tol):
    errs = {}
    for name, g, r, ax in zip(NAMES, got, ref, HEAD_AXIS):
        errs[name] = assert_close(name, g, r, tol, head_axis=ax)
    return errs


@pytest.mark.parametrize("B,T,H,D,dtype,s_in,ds,decay,seg", [
    (1, 256, 2, 64, "f32", None, 0.1, 1.0, 0),
    (1, 256, 2, 64, "f32", 0.1, 0.1, 0.01, 1),
    (2, 333, 2, 64, "f32", 0.1, 0.1, 0.01, 2),     # ragged, B = 2
    (1, 256, 2, 128, "f32", None, 0.1, 1.0, 0),    # fp32 at d = 128
    (2, 333, 2, 128, "f32", 0.1, 0.1, 0.01, 2),    # fp32 at d = 128: ragged, B = 2
    (1, 1000, 2, 128, "f32", 0.1, 0.1, 0.01, 3),   # fp32 at d = 128: ragged segments
    (1, 1000, 3, 128, "bf16", 0.1, 0.1, 0.01, 0),  # ragged, several segments
    (1, 640, 2, 128, "bf16", None, 0.1, 1.0, 3),
    (1, 1, 2, 128, "bf16", 0.1, 0.1, 1.0, 0),      # single token
    (1, 65, 2, 64, "bf16", 0.1, None, 0.01, 1),    # no exit gradient
    (2, 2048, 2, 128, "bf16", 0.1, 0.1, 0.01, 5),
    (1, 1000, 2, 64, "bf16", 0.1, 0.1, 0.01, 5),   # d = 64: segments of 5, 5, 5, 1 blocks
])
def test_bwd_matches_oracle(oracle_mod, B, T, H, D, dtype, s_in, ds, decay, seg):
    d = inputs(B, T, H, D, dtype, seed=2000 + T + H, s_in_std=s_in, grads=True, decay=decay,
               ds_std=ds)
    got = run_bwd(d, seg)
    ref = oracle_bwd(oracle_mod, d)
    check_all(got, ref, TOL[dtype])


def test_full_size_t16384_sampled_heads(oracle_mod):
    """H=16, T=16384, d=128, bf16, dO ~ N(0,1), dS_out ~ N(0,0.1), S_in = 0, in
    the launch configuration the benchmark uses; four heads checked whole."""
    d = inputs(1, 16384, 16, 128, "bf16", seed=20260003, grads=True)
    got = run_bwd(d)
    hs = [0, 5, 10, 15]
    sub = head_slice(d, hs)
    ref = oracle_bwd(oracle_mod, sub)
    sel = [g[:, :, hs] if ax == 2 else g[:, hs] for g, ax in zip(got, HEAD_AXIS)]
    check_all(sel, ref, TOL["bf16"])


def test_full_size_t16384_nonzero_state_sampled(oracle_mod):
    """Supplementary run with S_in ~ N(0, 0.1) so dalpha sees the entry state."""
    d = inputs(1, 16384, 16, 128, "bf16", seed=20260013, s_in_std=0.1, grads=True, decay=0.01)
    got = run_bwd(d)
    hs = [3, 8, 12]
    sub = head_slice(d, hs)
    ref = oracle_bwd(oracle_mod, sub)
    sel = [g[:, :, hs] if ax == 2 else g[:, hs] for g, ax in zip(got, HEAD_AXIS)]
    check_all(sel, ref, TOL["bf16"])


def _fd_probe(oracle_mod, d, got, tol=2e-2):
    """Directional derivatives of L = <dO, o> + <dS_out, S_out>: central
    differences of the fp64 oracle forward against the device gradient, for
    each input x along (a) the device gradient's own direction and (b) the
    unit vector of its largest coordinate.  (a) checks |grad| and its sign,
    (b) one large element; both compare relative to the finite difference
    itself, so a flipped or rescaled gradient fails."""
    base = {k: as_f64(d[k]) for k in ("q", "k", "v", "alpha", "beta", "S_in")}
    dO, dS = as_f64(d["dO"]), as_f64(d["dS_out"])

    def loss(x):
        o, S = oracle_mod.gdn_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S_in"])
        return float(np.sum(dO * o) + np.sum(dS * S))

    gname = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "S_in": "dS_in"}
    for name, x in base.items():
        g = got[gname[name]]
        dirs = [g / np.linalg.norm(g)]
        e = np.zeros_like(x)
        e.flat[int(np.argmax(np.abs(g)))] = 1.0
        dirs.append(e)
        for j, u in enumerate(dirs):
            h = 1e-6 * max(1.0, np.abs(x).max())
            xp, xm = dict(base), dict(base)
            xp[name] = x + h * u
            xm[name] = x - h * u
            fd = (loss(xp) - loss(xm)) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= tol * abs(fd) + 1e-9, (name, j, fd, an)


def test_finite_difference_probe(oracle_mod):
    d = inputs(1, 512, 2, 64, "bf16", seed=77, s_in_std=0.1, grads=True, decay=0.05)
    _fd_probe(oracle_mod, d, dict(zip(NAMES, run_bwd(d))))


def test_finite_difference_probe_t16384_head(oracle_mod):
    """The probe on one head of the H=16, T=16384, d=128 fwd+bwd workload
    (S_in ~ N(0, 0.1), slow decay so that every term of the gradient is
    exercised), with the gradients of the full-size device run."""
    d = inputs(1, 16384, 16, 128, "bf16", seed=20260023, s_in_std=0.1, grads=True, decay=0.01)
    got = run_bwd(d)
    hs = [5]
    sub = head_slice(d, hs)
    sel = [g[:, :, hs] if ax == 2 else g[:, hs] for g, ax in zip(got, HEAD_AXIS)]
    _fd_probe(oracle_mod, sub, dict(zip(NAMES, sel)))


def test_chained_nonuniform_fwd_bwd(oracle_mod):
    """Eight skewed chunks (the c_i(0.5) hybrid-cost plan, scaled to T=16384)
    chained forward (Eq. 5) then backward (Eq. 7) against the unchunked
    oracle."""
    T = 16384
    lengths = chunk_lengths(T, 8, 0.5)
    d = inputs(1, T, 4, 128, "bf16", seed=20260004, grads=True, decay=0.01)
    dd = to_dev(d)
    o, states = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None, lengths)
    g = gdn.chain_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["dO"], dd["dS_out"],
                      lengths, states)
    torch.cuda.synchronize()
    ref = oracle_bwd(oracle_mod, d)
    check_all([f64(x) for x in g], ref, TOL["bf16"])
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(states[-1]), S_ref, TOL["bf16"], head_axis=1)


def test_bwd_deterministic():
    d = to_dev(inputs(1, 3000, 3, 128, "bf16", seed=9, s_in_std=0.1, grads=True))
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"], d["dO"], d["dS_out"])
    r1 = gdn.chunk_bwd(*args)
    r2 = gdn.chunk_bwd(*args)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_bwd_empty_chunk_passes_gradient():
    d = to_dev(inputs(1, 0, 2, 64, "bf16", seed=10, s_in_std=0.1, grads=True))
    r = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"], d["dO"],
                      d["dS_out"])
    torch.cuda.synchronize()
    assert torch.equal(r[5], d["dS_out"])


@pytest.mark.parametrize("B,T,H,D,dtype,seg,decay", [
    (1, 256, 2, 64, "f32", 1, 0.01),
    (2, 333, 2, 64, "f32", 2, 0.01),      # ragged, B = 2
    (2, 333, 2, 128, "f32", 2, 0.01),     # fp32 at d = 128: ragged, B = 2
    (1, 1000, 3, 128, "bf16", 0, 0.01),   # ragged, several segments
    (1, 640, 2, 128, "bf16", 100, 0.01),  # one segment
    (1, 1, 2, 128, "bf16", 0, 1.0),       # single token (as in the oracle test above)
    (2, 2048, 2, 128, "bf16", 5, 0.01),
])
def test_saved_path_bitwise_equals_recompute(oracle_mod, B, T, H, D, dtype, seg, decay):
    """The saving forward returns the plain forward's o and S_out, and the
    saved backward the recompute backward's gradients, bit for bit; both
    also against the oracle."""
    d = inputs(B, T, H, D, dtype, seed=3000 + T, s_in_std=0.1, grads=True, decay=decay)
    dd = to_dev(d)
    fa = (dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
    o1, S1 = gdn.chunk_fwd(*fa, seg_blocks=seg)
    o2, S2, saved = gdn.chunk_fwd(*fa, seg_blocks=seg, saved=True)
    g1 = gdn.chunk_bwd(*fa, dd["dO"], dd["dS_out"], seg_blocks=seg)
    g2 = gdn.chunk_bwd(*fa[:5], None, dd["dO"], dd["dS_out"], seg_blocks=seg, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for name, x, y in zip(NAMES, g1, g2):
        assert torch.equal(x, y), name
    check_all([f64(x) for x in g2], oracle_bwd(oracle_mod, d), TOL[dtype])


def test_saved_buffer_reused_across_shapes():
    """One saved buffer sized for the larger chunk serves a smaller one."""
    big = to_dev(inputs(1, 4096, 2, 128, "bf16", seed=31, s_in_std=0.1, grads=True))
    small = to_dev(inputs(1, 700, 2, 128, "bf16", seed=32, s_in_std=0.1, grads=True))
    _, _, saved = gdn.chunk_fwd(big["q"], big["k"], big["v"], big["alpha"], big["beta"],
                                big["S_in"], saved=True)
    for dd in (small, big):
        fa = (dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
        gdn.chunk_fwd(*fa, saved=saved)
        g1 = gdn.chunk_bwd(*fa, dd["dO"], dd["dS_out"])
        g2 = gdn.chunk_bwd(*fa[:5], None, dd["dO"], dd["dS_out"], saved=saved)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, g1, g2):
            assert torch.equal(x, y), name


def test_fp32_d128_chain_fwd_bwd(oracle_mod):
    """fp32 at d = 128, chained over three uneven chunks (Eqs. 5 and 7), the
    saving forward and the saved backward, against the unchunked oracle at
    the fp32 bar.  8 heads x 64 blocks in the largest chunk: more blocks
    than the gradient kernel's workgroups, so each workgroup takes several."""
    T = 4096 + 1000
    lengths = [4096, 640, 360]
    d = inputs(1, T, 8, 128, "f32", seed=20260020, s_in_std=0.1, grads=True, decay=0.01)
    dd = to_dev(d)
    o, states, saved = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"],
                                     dd["S_in"], lengths, save=True)
    g = gdn.chain_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["dO"],
                      dd["dS_out"], lengths, None, saved=saved)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["f32"], head_axis=2)
    assert_close("S_out", f64(states[-1]), S_ref, TOL["f32"], head_axis=1)
    check_all([f64(x) for x in g], oracle_bwd(oracle_mod, d), TOL["f32"])


def test_saved_chain_nonuniform_fwd_bwd(oracle_mod):
    """The skewed eight-chunk chain of the test above through the saving
    forward and the saved backward."""
    T = 16384
    lengths = chunk_lengths(T, 8, 0.5)
    d = inputs(1, T, 4, 128, "bf16", seed=20260004, grads=True, decay=0.01)
    dd = to_dev(d)
    o, states, saved = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None,
                                     lengths, save=True)
    g = gdn.chain_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["dO"],
                      dd["dS_out"], lengths, None, saved=saved)
    torch.cuda.synchronize()
    check_all([f64(x) for x in g], oracle_bwd(oracle_mod, d), TOL["bf16"])


def test_full_size_benchmark_chain_sampled_heads(oracle_mod):
    """The benchmark workload at its full size and in the launch
    configuration the benchmark times: T = 262,144, H = 16, d = 128, bf16,
    eight chunks by the c_i(0.5) plan, the saving forward then the saved
    backward, chained.  Inputs are drawn on the device by the seeded
    generator, as the benchmark draws them; four heads are copied out and
    checked whole against the unchunked oracle (chunking is exact in real
    arithmetic), forward and backward."""
    T, H = 262144, 16
    lengths = chunk_lengths(T, 8, 0.5)
    dd = inputs(1, T, H, 128, "bf16", seed=20260004, grads=True, device="cuda")
    o, states, saved = gdn.chain_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None,
                                     lengths, save=True)
    g = gdn.chain_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["dO"],
                      dd["dS_out"], lengths, None, saved=saved)
    torch.cuda.synchronize()
    hs = [1, 6, 9, 14]
    sub = head_slice(dd, hs)
    o_ref, s_ref = oracle_mod.gdn_fwd(*oracle_args(sub))
    assert_close("o", f64(o[:, :, hs]), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(states[-1][:, hs]), s_ref, TOL["bf16"], head_axis=1)
    ref = oracle_bwd(oracle_mod, sub)
    sel = [f64(x[:, :, hs]) if ax == 2 else f64(x[:, hs]) for x, ax in zip(g, HEAD_AXIS)]
    check_all(sel, ref, TOL["bf16"])


def test_saved_bwd_empty_chunk():
    d = to_dev(inputs(1, 0, 2, 64, "bf16", seed=10, s_in_std=0.1, grads=True))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    o, S, saved = gdn.chunk_fwd(*fa, saved=True)
    r = gdn.chunk_bwd(*fa[:5], None, d["dO"], d["dS_out"], saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(S, d["S_in"])
    assert torch.equal(r[5], d["dS_out"])


# Short chunks with slow decay and a carried state (alpha = exp(-0.01
# softplus(N(0,1))), S_in ~ N(0, 0.1)): the boundary state enters every
# output and gradient.  Forward and backward, recompute and saved paths.
SHORT = [(T, D, dt) for T in (1, 2, 65) for D in (64, 128) for dt in ("bf16",)] + \
        [(T, D, "f32") for T in (1, 2, 65) for D in (64, 128)]


def _short_case(T, D, dtype, saved):
    d = inputs(1, T, 4, D, dtype, seed=9100 + 7 * T + D, s_in_std=0.1, grads=True, decay=0.01)
    dd = to_dev(d)
    fa = (dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
    if saved:
        o, S, sv = gdn.chunk_fwd(*fa, saved=True)
        g = gdn.chunk_bwd(*fa[:5], None, dd["dO"], dd["dS_out"], saved=sv)
    else:
        o, S = gdn.chunk_fwd(*fa)
        g = gdn.chunk_bwd(*fa, dd["dO"], dd["dS_out"])
    torch.cuda.synchronize()
    return d, f64(o), f64(S), [f64(x) for x in g]


@pytest.mark.parametrize("saved", [False, True])
@pytest.mark.parametrize("T,D,dtype", SHORT)
def test_short_chunks_slow_decay(oracle_mod, T, D, dtype, saved):
    """Every output per head.  For bf16 chunks of one or two tokens a head's
    dalpha and dbeta are one or two values (the per-head bar is then an
    elementwise relative error); such chunks, like every bf16 chunk of one
    64-token block, run on the fp32 kernels over upcast inputs.  On the bf16
    kernels they missed by up to 9.6e-2 (dalpha) and 5.0e-2 (dbeta) relative
    to that value."""
    d, o, S, got = _short_case(T, D, dtype, saved)
    tol = TOL[dtype]
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", o, o_ref, tol, head_axis=2)
    assert_close("S_out", S, S_ref, tol, head_axis=1)
    ref = oracle_bwd(oracle_mod, d)
    for name, g, r, ax in zip(NAMES, got, ref, HEAD_AXIS):
        assert_close(name, g, r, tol, head_axis=ax)


@pytest.mark.parametrize("saved", [False, True])
@pytest.mark.parametrize("T,D", [(1, 64), (2, 128), (64, 128)])
def test_one_block_bf16_runs_fp32(oracle_mod, T, D, saved):
    """A bf16 chunk of one block matches the oracle far inside the bf16 bar:
    its products run in fp32 on the exact bf16 inputs, so only the final
    rounding of o, dq, dk, dv to bf16 remains (about 2^-9 of each value) and
    the fp32 outputs (S_out, the gate gradients, dS_in) are within 1e-4."""
    d, o, S, got = _short_case(T, D, "bf16", saved)
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", o, o_ref, 4e-3, head_axis=2)
    assert_close("S_out", S, S_ref, TOL["f32"], head_axis=1)
    ref = oracle_bwd(oracle_mod, d)
    for name, g, r, ax in zip(NAMES, got, ref, HEAD_AXIS):
        tol = 4e-3 if name in ("dq", "dk", "dv") else TOL["f32"]
        assert_close(name, g, r, tol, head_axis=ax)

def test_one_block_bf16_two_batches(oracle_mod):
    """The same with B = 2, three heads and a ragged block (37 tokens), d = 64,
    recompute path, and S_in ~ N(0, 0.1) with slow decay."""
    d = inputs(2, 37, 3, 64, "bf16", seed=9300, s_in_std=0.1, grads=True, decay=0.01)
    dd = to_dev(d)
    fa = (dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
    o, S = gdn.chunk_fwd(*fa)
    g = gdn.chunk_bwd(*fa, dd["dO"], dd["dS_out"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, 4e-3, head_axis=2)
    assert_close("S_out", f64(S), S_ref, TOL["f32"], head_axis=1)
    for name, x, r, ax in zip(NAMES, g, oracle_bwd(oracle_mod, d), HEAD_AXIS):
        assert_close(name, f64(x), r, 4e-3 if name in ("dq", "dk", "dv") else TOL["f32"],
                     head_axis=ax)


def test_single_head_long_chunk(oracle_mod):
    """One sequence (B = H = 1) of 65,537 tokens at d = 128, bf16, slow decay
    and a carried state, in the default plan: 57 segments of 18 blocks, so
    the segment chains run 56 steps on a grid that is mostly padding
    workgroups, and the last block holds one token.  Forward and backward,
    whole, against the oracle."""
    d = inputs(1, 65537, 1, 128, "bf16", seed=20261201, s_in_std=0.1, grads=True, decay=0.01)
    from linear_recurrence_chunked_gated_amd import _lib
    assert _lib.segment_plan(_lib.make_shape(1, 65537, 1, 128, 128, torch.bfloat16)) == (18, 57)
    dd = to_dev(d)
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(S), S_ref, TOL["bf16"], head_axis=1)
    check_all(run_bwd(d), oracle_bwd(oracle_mod, d), TOL["bf16"])
