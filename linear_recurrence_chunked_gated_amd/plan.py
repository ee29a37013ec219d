"""Nonuniform pipeline-chunk lengths from the hybrid cost model.

Source: "Pith review of StateFlow: Sequence Pipeline Parallelism for
Long-Context Modeling with Linear Recurrence", "What carries the argument":
a chunk starting at token c_i with s_i tokens costs (Eq. 9)

    Cost_i = a s_i + b (c_i s_i + s_i^2 / 2),   a = L_lin C_lin + C_dense,
                                                b = L_soft C_soft,

and the equal-cost boundaries c_i^hybrid are blended with the uniform ones,
c_i(alpha) = (1 - alpha) c_i^equal + alpha c_i^hybrid.

Eq. 9 telescopes: Cost_i = F(c_{i+1}) - F(c_i) with F(x) = a x + b x^2 / 2,
so the equal-cost boundary solves the quadratic F(c_i) = (i / N) F(T) and has
the closed form used below.  Inner boundaries are rounded to the nearest
multiple of the kernel block so that every chunk is whole blocks.
"""
import math


def hybrid_boundary(i, T, N, a, b):
    """c_i^hybrid: the root of b/2 c^2 + a c - (i/N) F(T) = 0 in [0, T]."""
    if b == 0.0:
        return i * T / N
    y = (i / N) * (a * T + 0.5 * b * T * T)
    return (-a + math.sqrt(a * a + 2.0 * b * y)) / b


def chunk_lengths(T, N, alpha, a=1.0, b=0.25, multiple=64):
    """Lengths of N chunks for c_i(alpha), inner boundaries rounded to the
    nearest multiple of ``multiple`` (ties round up)."""
    if T % multiple:
        raise ValueError("T must be a multiple of %d" % multiple)
    bounds = [0]
    for i in range(1, N):
        c = (1.0 - alpha) * i * T / N + alpha * hybrid_boundary(i, T, N, a, b)
        bounds.append(int(math.floor(c / multiple + 0.5)) * multiple)
    bounds.append(T)
    lengths = [bounds[i + 1] - bounds[i] for i in range(N)]
    if min(lengths) <= 0:
        raise ValueError("degenerate partition %r" % (lengths,))
    return lengths
