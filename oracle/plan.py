"""TEST INFRASTRUCTURE: plain search for nonuniform chunk boundaries.

Source: "Pith review of StateFlow: Sequence Pipeline Parallelism for
Long-Context Modeling with Linear Recurrence", "What carries the argument":
the hybrid cost model (Eq. 9)

    Cost_i = (L_lin C_lin + C_dense) s_i + L_soft C_soft (c_i s_i + s_i^2 / 2)

for a chunk that starts at token c_i and holds s_i tokens, whose equal-cost
solution c_i^hybrid anchors the family c_i(alpha) = (1 - alpha) c_i^equal +
alpha c_i^hybrid.  The page leaves the coefficients open; the caller passes
them.

This module finds each equal-cost boundary by bisection on Eq. 9 itself, one
chunk after the other, so it shares nothing with the closed-form planner in
the product.
"""


def chunk_cost(c, s, lin, soft):
    """Eq. 9 for one chunk starting at c with s tokens."""
    return lin * s + soft * (c * s + s * s / 2.0)


def hybrid_boundaries(T, N, lin, soft, iters=200):
    """Real-valued boundaries 0 = c_0 < ... < c_N = T with equal Eq. 9 cost."""
    total = chunk_cost(0.0, float(T), lin, soft)
    target = total / N
    bounds = [0.0]
    c = 0.0
    for _ in range(N - 1):
        lo, hi = c, float(T)
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            if chunk_cost(c, mid - c, lin, soft) < target:
                lo = mid
            else:
                hi = mid
        c = 0.5 * (lo + hi)
        bounds.append(c)
    bounds.append(float(T))
    return bounds


def skewed_lengths(T, N, alpha, lin, soft, multiple):
    """Chunk lengths for c_i(alpha), with each inner boundary rounded to the
    nearest multiple of ``multiple`` (c_0 = 0 and c_N = T are kept)."""
    hyb = hybrid_boundaries(T, N, lin, soft)
    bounds = [0]
    for i in range(1, N):
        ci = (1.0 - alpha) * (i * T / N) + alpha * hyb[i]
        q = int(ci // multiple)
        rem = ci - q * multiple
        bounds.append((q + 1) * multiple if rem >= multiple / 2.0 else q * multiple)
    bounds.append(T)
    return [bounds[i + 1] - bounds[i] for i in range(N)]
