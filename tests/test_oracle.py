"""Pins for the fp64 CPU oracle, independent of its own code.

Each test checks the oracle against something the mathematics fixes:
a hand-worked example, exact rational brute force with explicit transition
matrices, closed forms of special cases, a textbook reduction (causal linear
attention), an independent chunkwise (WY/UT) algorithm, automatic and finite
differentiation, and the chunk-chaining identity (Eqs. 5 and 7 of the
StateFlow page, "What carries the argument").
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, Dk, Dv, unit_keys=True, s_in=True, decay=1.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    alpha = np.exp(-decay * np.logaddexp(0.0, rng.standard_normal((B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S_in = 0.3 * rng.standard_normal((B, H, Dv, Dk)) if s_in else None
    return q, k, v, alpha, beta, S_in


# ---------------------------------------------------------------- golden ---

def _frac(x):
    if isinstance(x, list):
        return [_frac(e) for e in x]
    return Fraction(x)


def _f(x):
    return np.array(_frac(x), dtype=object).astype(float)


def test_hand_worked_example(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_d2_t2.json")) as f:
        g = json.load(f)
    inp, exp = g["inputs"], g["expected"]
    q = _f(inp["q"]).reshape(1, 2, 1, 2)
    k = _f(inp["k"]).reshape(1, 2, 1, 2)
    v = _f(inp["v"]).reshape(1, 2, 1, 2)
    a = _f(inp["alpha"]).reshape(1, 2, 1)
    b = _f(inp["beta"]).reshape(1, 2, 1)
    S0 = _f(inp["S_in"]).reshape(1, 1, 2, 2)
    dO = _f(inp["dO"]).reshape(1, 2, 1, 2)
    dS = _f(inp["dS_out"]).reshape(1, 1, 2, 2)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    np.testing.assert_allclose(o.reshape(2, 2), _f(exp["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(S.reshape(2, 2), _f(exp["S_out"]), rtol=0, atol=1e-15)
    dq, dk, dv, da, db, dS0 = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dS)
    np.testing.assert_allclose(dq.reshape(2, 2), _f(exp["dq"]), atol=1e-15)
    np.testing.assert_allclose(dk.reshape(2, 2), _f(exp["dk"]), atol=1e-15)
    np.testing.assert_allclose(dv.reshape(2, 2), _f(exp["dv"]), atol=1e-15)
    np.testing.assert_allclose(da.reshape(2), _f(exp["dalpha"]), atol=1e-15)
    np.testing.assert_allclose(db.reshape(2), _f(exp["dbeta"]), atol=1e-15)
    np.testing.assert_allclose(dS0.reshape(2, 2), _f(exp["dS_in"]), atol=1e-15)


# ------------------------------------------------- exact brute force -------

def _mat_mul(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def _brute_force_exact(q, k, v, a, b, S0):
    """Explicit d x d transition matrices in exact rational arithmetic:
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t."""
    T = len(a)
    Dk = len(k[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        Mt = [[(Fraction(1) if i == j else Fraction(0)) - b[t] * k[t][i] * k[t][j]
               for j in range(Dk)] for i in range(Dk)]
        SM = _mat_mul(S, Mt)
        S = [[a[t] * SM[i][j] + b[t] * v[t][i] * k[t][j] for j in range(Dk)]
             for i in range(len(S))]
        outs.append([sum(S[i][j] * q[t][j] for j in range(Dk)) for i in range(len(S))])
    return outs, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_brute_force(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    T, Dk, Dv = 5, 3, 2

    def dy(shape, lo, hi, den):  # dyadic rationals: exact in fp64
        return [Fraction(int(x), den) for x in rng.integers(lo, hi, size=shape).ravel()]

    qf = dy((T, Dk), -16, 17, 16)
    kf = dy((T, Dk), -16, 17, 16)
    vf = dy((T, Dv), -16, 17, 8)
    af = dy((T,), 1, 33, 32)
    bf = dy((T,), 0, 33, 32)
    S0f = dy((Dv, Dk), -8, 9, 8)
    q = [qf[t * Dk:(t + 1) * Dk] for t in range(T)]
    k = [kf[t * Dk:(t + 1) * Dk] for t in range(T)]
    v = [vf[t * Dv:(t + 1) * Dv] for t in range(T)]
    S0 = [S0f[i * Dk:(i + 1) * Dk] for i in range(Dv)]
    outs, S = _brute_force_exact(q, k, v, af, bf, S0)
    fl = lambda x: np.array(x, dtype=object).astype(float)
    o_or, S_or = oracle_mod.gdn_fwd(fl(q).reshape(1, T, 1, Dk), fl(k).reshape(1, T, 1, Dk),
                                    fl(v).reshape(1, T, 1, Dv), fl(af).reshape(1, T, 1),
                                    fl(bf).reshape(1, T, 1), fl(S0).reshape(1, 1, Dv, Dk))
    np.testing.assert_allclose(o_or.reshape(T, Dv), fl(outs), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S_or.reshape(Dv, Dk), fl(S), rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- closed forms ------

def test_beta_zero_is_pure_decay(oracle_mod):
    rng = np.random.default_rng(3)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 37, 3, 5, 4)
    b[:] = 0.0
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    cum = np.cumprod(a, axis=1)  # [B,T,H]
    ref = np.einsum("bth,bhij,bthj->bthi", cum, S0, q)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, cum[:, -1, :, None, None] * S0, rtol=1e-12, atol=1e-14)


def test_single_token_from_zero(oracle_mod):
    rng = np.random.default_rng(4)
    q, k, v, a, b, _ = rand_inputs(rng, 1, 1, 2, 6, 5)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, None)
    ref = b[..., None] * np.sum(k * q, -1, keepdims=True) * v
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S[0], b[0, 0][:, None, None] * v[0, 0][:, :, None] * k[0, 0][:, None, :],
                               rtol=1e-13, atol=1e-15)


def test_identity_gate_keeps_state(oracle_mod):
    rng = np.random.default_rng(5)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 20, 2, 4, 4)
    a[:] = 1.0
    b[:] = 0.0
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("bhij,bthj->bthi", S0, q), rtol=1e-13, atol=1e-15)


def test_full_write_overwrites_key_direction(oracle_mod):
    # beta = 1 and |k| = 1: S_t k_t = v_t whatever S_{t-1} and alpha are.
    rng = np.random.default_rng(6)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 12, 2, 8, 8)
    b[:] = 1.0
    for t in range(1, 13):
        _, S = oracle_mod.gdn_fwd(q[:, :t], k[:, :t], v[:, :t], a[:, :t], b[:, :t], S0)
        Sk = np.einsum("bhij,bhj->bhi", S, k[:, t - 1])
        np.testing.assert_allclose(Sk, v[:, t - 1], rtol=1e-12, atol=1e-12)


def test_reduces_to_causal_linear_attention(oracle_mod):
    # alpha = 1, beta = 1, S_0 = 0 and orthonormal keys: o_t = sum_{s<=t} v_s (k_s . q_t).
    rng = np.random.default_rng(7)
    Dk, Dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm.T[None, :, None, :].copy()          # rows are orthonormal
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    a = np.ones((1, T, 1))
    b = np.ones((1, T, 1))
    o, _ = oracle_mod.gdn_fwd(q, k, v, a, b, None)
    scores = np.tril(q[0, :, 0] @ k[0, :, 0].T)   # [t, s]
    ref = scores @ v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------ independent chunkwise algebra --

def chunkwise_fwd_np(q, k, v, alpha, beta, S_in, C):
    """WY/UT block form, written independently of the oracle (dense solve
    for the unit-lower system)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    S_out = np.zeros((B, H, Dv, Dk))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((Dv, Dk)) if S_in is None else S_in[bb, h].copy()
            for t0 in range(0, T, C):
                sl = slice(t0, min(T, t0 + C))
                Q, K, V = q[bb, sl, h], k[bb, sl, h], v[bb, sl, h]
                g = np.cumsum(np.log(alpha[bb, sl, h]))
                be = beta[bb, sl, h]
                n = len(g)
                Gam = np.tril(np.exp(g[:, None] - g[None, :]))
                A = np.tril(be[:, None] * (K @ K.T) * Gam, -1)
                Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
                W = Tm @ ((be * np.exp(g))[:, None] * K)
                U = Tm @ (be[:, None] * V)
                Vn = U - W @ S.T
                o[bb, sl, h] = np.exp(g)[:, None] * (Q @ S.T) + np.tril(Q @ K.T * Gam) @ Vn
                S = np.exp(g[-1]) * S + Vn.T @ (np.exp(g[-1] - g)[:, None] * K)
            S_out[bb, h] = S
    return o, S_out


@pytest.mark.parametrize("T,C,decay", [(64, 16, 1.0), (150, 32, 1.0), (150, 64, 0.01), (9, 4, 0.01)])
def test_matches_independent_chunkwise_form(oracle_mod, T, C, decay):
    rng = np.random.default_rng(8 + T)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, T, 2, 12, 10, decay=decay)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    o2, S2 = chunkwise_fwd_np(q, k, v, a, b, S0, C)
    scale_o = np.abs(o).max()
    assert np.abs(o - o2).max() <= 1e-12 * scale_o
    assert np.abs(S - S2).max() <= 1e-12 * np.abs(S).max()


# ------------------------------------------------------------- backward ----

def _torch_literal_loss_grads(q, k, v, a, b, S0, dO, dSo):
    """Autograd through the literal matrix form of the recurrence."""
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, b, S0)]
    tq, tk, tv, ta, tb, tS0 = ts
    B, T, H, Dk = q.shape
    loss = 0.0
    for bb in range(B):
        for h in range(H):
            S = tS0[bb, h]
            eye = torch.eye(Dk, dtype=torch.float64)
            for t in range(T):
                kt = tk[bb, t, h]
                S = ta[bb, t, h] * S @ (eye - tb[bb, t, h] * torch.outer(kt, kt)) \
                    + tb[bb, t, h] * torch.outer(tv[bb, t, h], kt)
                loss = loss + torch.dot(torch.tensor(dO[bb, t, h]), S @ tq[bb, t, h])
            loss = loss + torch.sum(torch.tensor(dSo[bb, h]) * S)
    loss.backward()
    return [x.grad.numpy() for x in ts]


def test_backward_matches_autograd_of_literal_form(oracle_mod):
    rng = np.random.default_rng(11)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 70, 2, 5, 4)
    dO = rng.standard_normal(q.shape[:3] + (4,))
    dSo = rng.standard_normal(S0.shape)
    dq, dk, dv, da, db, dS0 = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)
    ref = _torch_literal_loss_grads(q, k, v, a, b, S0, dO, dSo)
    for got, want in zip((dq, dk, dv, da, db, dS0), ref):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-11)


def test_backward_finite_differences(oracle_mod):
    rng = np.random.default_rng(12)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 150, 2, 8, 6, decay=0.05)
    dO = rng.standard_normal(v.shape)
    dSo = rng.standard_normal(S0.shape)

    def loss(q, k, v, a, b, S0):
        o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
        return float(np.sum(dO * o) + np.sum(dSo * S))

    grads = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)
    grads = dict(zip("q k v a b S0".split(), [grads[0], grads[1], grads[2], grads[3], grads[4], grads[5]]))
    base = dict(q=q, k=k, v=v, a=a, b=b, S0=S0)
    for name in base:
        d = rng.standard_normal(base[name].shape)
        d /= np.linalg.norm(d)
        h = 1e-6 * max(1.0, np.abs(base[name]).max())
        plus = dict(base)
        minus = dict(base)
        plus[name] = base[name] + h * d
        minus[name] = base[name] - h * d
        fd = (loss(**plus) - loss(**minus)) / (2 * h)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_closed_form_state_gradient_when_beta_zero(oracle_mod):
    # beta = 0: S_t = (prod_{j<=t} alpha_j) S_0, so
    # dS_in = (prod alpha) dS_out + sum_t (prod_{j<=t} alpha_j) dO_t q_t^T.
    rng = np.random.default_rng(13)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 30, 2, 4, 3, decay=0.1)
    b[:] = 0.0
    dO = rng.standard_normal(v.shape)
    dSo = rng.standard_normal(S0.shape)
    dq, dk, dv, da, db, dS0 = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)
    cum = np.cumprod(a, axis=1)
    ref = cum[:, -1, :, None, None] * dSo + np.einsum("bth,bthi,bthj->bhij", cum, dO, q)
    np.testing.assert_allclose(dS0, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, 0.0, atol=0)
    np.testing.assert_allclose(dk, 0.0, atol=0)


def test_dalpha_at_tiny_alpha_finite_differences(oracle_mod):
    """Strong decay (alpha = exp(-10 softplus(z)), down to about 1e-13).  Each
    state is affine in each alpha_t, and so is the loss, so a central
    difference in alpha_t is exact up to rounding for any step; a step of
    0.25 (the affine extension past alpha = 0 included) resolves dalpha at
    the tokens with the smallest alpha, where dalpha stays of the order of
    the other gradients while d log alpha = alpha dalpha vanishes."""
    rng = np.random.default_rng(14)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 80, 1, 6, 5, decay=10.0)
    dO = rng.standard_normal(v.shape)
    dSo = rng.standard_normal(S0.shape)
    da = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)[3]

    def loss(a):
        o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
        return float(np.sum(dO * o) + np.sum(dSo * S))

    order = np.argsort(a[0, :, 0])
    assert a[0, order[0], 0] < 1e-10
    scale = np.abs(da).max()
    for t in order[:6]:
        h = 0.25
        ap, am = a.copy(), a.copy()
        ap[0, t, 0] += h
        am[0, t, 0] -= h
        fd = (loss(ap) - loss(am)) / (2 * h)
        assert abs(fd - da[0, t, 0]) <= 1e-6 * scale, (t, a[0, t, 0], fd, da[0, t, 0])


def test_tiny_alpha_resets_the_state(oracle_mod):
    """With alpha_R = 1e-30 the state carried into token R is scaled away:
    from R on, outputs and the exit state equal those of the sequence
    restarted at R from a zero state, and the gradients of the tokens before
    R equal those of the prefix with no exit gradient (dalpha_R, which reads
    the state before R, excepted)."""
    rng = np.random.default_rng(15)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 90, 2, 5, 4, decay=0.3)
    R = 37
    a[:, R] = 1e-30
    dO = rng.standard_normal(v.shape)
    dSo = rng.standard_normal(S0.shape)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    o2, S2 = oracle_mod.gdn_fwd(q[:, R:], k[:, R:], v[:, R:], a[:, R:], b[:, R:], None)
    np.testing.assert_allclose(o[:, R:], o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-14)
    g = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)
    g1 = oracle_mod.gdn_bwd(q[:, :R], k[:, :R], v[:, :R], a[:, :R], b[:, :R], S0, dO[:, :R], None)
    g2 = oracle_mod.gdn_bwd(q[:, R:], k[:, R:], v[:, R:], a[:, R:], b[:, R:], None, dO[:, R:], dSo)
    for i in range(5):
        np.testing.assert_allclose(g[i][:, :R], g1[i], rtol=1e-12, atol=1e-14)
        if i == 3:
            np.testing.assert_allclose(g[i][:, R + 1:], g2[i][:, 1:], rtol=1e-12, atol=1e-14)
        else:
            np.testing.assert_allclose(g[i][:, R:], g2[i], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[5], g1[5], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- chaining ----

@pytest.mark.parametrize("lengths", [[64, 64, 64, 64], [10, 100, 1, 45]])
def test_chunk_chain_is_exact(oracle_mod, lengths):
    """Eq. 5 forward and Eq. 7 backward chaining reproduce the unchunked
    token loop bit for bit (same operations in the same order)."""
    rng = np.random.default_rng(14)
    T = sum(lengths)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, T, 2, 6, 5, decay=0.05)
    dO = rng.standard_normal(v.shape)
    dSo = rng.standard_normal(S0.shape)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    oc, Sc, _ = oracle_mod.gdn_fwd_chained(q, k, v, a, b, S0, lengths)
    np.testing.assert_array_equal(o, oc)
    np.testing.assert_array_equal(S, Sc)
    g = oracle_mod.gdn_bwd(q, k, v, a, b, S0, dO, dSo)
    gc = oracle_mod.gdn_bwd_chained(q, k, v, a, b, S0, dO, dSo, lengths)
    for x, y in zip(g, gc):
        np.testing.assert_array_equal(x, y)


def test_empty_sequence_passes_state_through(oracle_mod):
    rng = np.random.default_rng(15)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 0, 2, 4, 4)
    o, S = oracle_mod.gdn_fwd(q, k, v, a, b, S0)
    assert o.shape == (1, 0, 2, 4)
    np.testing.assert_array_equal(S, S0)
    dSo = rng.standard_normal(S0.shape)
    r = oracle_mod.gdn_bwd(q, k, v, a, b, S0, np.zeros((1, 0, 2, 4)), dSo)
    np.testing.assert_array_equal(r[5], dSo)


# ------------------------------------------------------------- planner -----

def test_oracle_planner_equal_cost():
    from oracle import plan as op
    T, N, lin, soft = 262144, 8, 1.0, 0.25
    hyb = op.hybrid_boundaries(T, N, lin, soft)
    costs = [op.chunk_cost(hyb[i], hyb[i + 1] - hyb[i], lin, soft) for i in range(N)]
    total = op.chunk_cost(0.0, T, lin, soft)
    np.testing.assert_allclose(costs, total / N, rtol=1e-9)
    # alpha = 0 is the uniform split; soft = 0 makes the hybrid split uniform.
    assert op.skewed_lengths(T, N, 0.0, lin, soft, 64) == [T // N] * N
    assert op.skewed_lengths(T, N, 1.0, lin, 0.0, 64) == [T // N] * N
