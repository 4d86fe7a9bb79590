"""Pins of the partition oracle: closed forms and a hand-worked case."""
import random
from fractions import Fraction

import pytest

from oracle.partition import partition_bruteforce, variance


def test_uniform_costs_split_evenly():
    for L, K in [(8, 2), (8, 4), (12, 3), (16, 16), (9, 1)]:
        b, v = partition_bruteforce([3.0] * L, K)
        assert b == list(range(0, L + 1, L // K))
        assert v == 0


def test_trivial_k():
    costs = [5, 1, 4, 2, 8]
    assert partition_bruteforce(costs, 1) == ([0, 5], 0)
    b, v = partition_bruteforce(costs, 5)
    assert b == [0, 1, 2, 3, 4, 5]
    assert v == variance(costs)


def test_hand_worked_case():
    # costs 1..6, prefix sums 1,3,6,10,15,21.  K=2: cells 10 | 11, variance 1/4.
    # K=3: cells 6 | 9 | 6 (mean 7), variance (1+4+1)/3 = 2; every other split is worse.
    assert partition_bruteforce([1, 2, 3, 4, 5, 6], 2) == ([0, 4, 6], Fraction(1, 4))
    assert partition_bruteforce([1, 2, 3, 4, 5, 6], 3) == ([0, 3, 5, 6], Fraction(2))


def test_variance_equals_sum_of_squares_form():
    rng = random.Random(4)
    for _ in range(50):
        cs = [rng.randint(0, 100) for _ in range(rng.randint(1, 7))]
        k = len(cs)
        assert variance(cs) == (Fraction(sum(c * c for c in cs)) - Fraction(sum(cs)) ** 2 / k) / k


def test_ties_take_lexicographically_smallest():
    # [1,1,1,1] with K=3 -> cells (2,1,1), (1,2,1), (1,1,2) tie; smallest bounds win.
    assert partition_bruteforce([1, 1, 1, 1], 3)[0] == [0, 1, 2, 4]


def test_invalid():
    with pytest.raises(ValueError):
        partition_bruteforce([1, 2], 3)
