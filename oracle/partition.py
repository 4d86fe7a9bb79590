"""Oracle for the cell partition (test infrastructure only).

GPipe splits a sequence of L layers, each with an estimated cost c_i, into K
contiguous cells and balances them by minimising the variance of the cells'
estimated costs (GPipe technical review page, "GPipe algorithm in detail /
minimal interface design").  The pages leave the search open; the plain
definition is used here: try every split into K non-empty contiguous cells
and keep the one of least variance, ties going to the lexicographically
smallest boundary vector.  Exact rational arithmetic makes ties exact.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import combinations


def variance(cell_costs):
    """Population variance (1/K) * sum_k (C_k - mean)^2, exactly."""
    cs = [Fraction(c) for c in cell_costs]
    mean = sum(cs) / len(cs)
    return sum((c - mean) ** 2 for c in cs) / len(cs)


def cell_costs(costs, bounds):
    return [sum(Fraction(c) for c in costs[bounds[k]:bounds[k + 1]])
            for k in range(len(bounds) - 1)]


def partition_bruteforce(costs, k):
    """Returns (bounds, variance): bounds[0]=0 < ... < bounds[K]=L."""
    n = len(costs)
    if not 1 <= k <= n:
        raise ValueError("need 1 <= K <= L")
    best = None
    for cuts in combinations(range(1, n), k - 1):   # lexicographic order
        bounds = (0,) + cuts + (n,)
        v = variance(cell_costs(costs, bounds))
        if best is None or v < best[1]:
            best = (list(bounds), v)
    return best[0], best[1]
