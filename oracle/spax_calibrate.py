"""Plain CPU oracle of the offline tier-size calibration (SpAx page, section
5.2: the read budget of Eq. 5, Step 1's greedy search over group budgets and
Step 2's grid over (k_top, k_mid)).

TEST INFRASTRUCTURE, like spax_oracle: only tests/ and the benchmark's CPU leg
may import it; it shares no code with the library's calibration module.

Readings (the page's Eq. 3 and Appendix B are not available):
  * Budgets are integer percentages; Step 1 lowers a group by 5 points
    (0.05 of its dense size).
  * A group's error is the l2 output error summed over its calibration
    tokens and its matrices: sum_t ||y_tiered(x_t) - W x_t||^2, with W x_t
    the dense product. Groups are evaluated on their own inputs, so a layer's
    error is the sum of its groups' errors, and Step 1's "reduction with the
    smallest l2 output error" is the one that raises that sum least (ties: the
    lower group index).
  * During Step 1 every group has k_mid = 0 (top-k at its budget):
    k_top = floor(budget n / 100).
  * Eq. 5 with rho = middle-tier bytes / top-tier bytes per column as an
    exact fraction: k_mid = min(n - k_top, floor((budget n / 100 - k_top) / rho)).
  * Step 2's grid: k_top_i = floor(k0 (S - i) / S), i = 0..S, from k0 =
    floor(budget n / 100); the walk stops after the first point whose bottom
    tier is empty (k_top + k_mid = n) or whose top tier is empty. The chosen
    setting is the first one with the smallest error.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

from .spax_oracle import ColumnStore, plan_tiers, tiered_product

__all__ = ["k_mid_for", "grid_points", "group_error", "step2_grid", "layer_budget",
           "step1_greedy"]


def k_mid_for(n: int, budget_pct: int, rho: Fraction, k_top: int) -> int:
    """Middle-tier columns that fill the budget left by k_top (Eq. 5)."""
    room = Fraction(budget_pct * n, 100) - k_top
    if room <= 0:
        return 0
    return int(min(n - k_top, room / rho))


def grid_points(n: int, budget_pct: int, rho: Fraction, steps: int) -> List[Tuple[int, int]]:
    """Step 2's grid: k_top lowered in equal steps from the all-top setting,
    k_mid raised to keep the budget, until a tier runs empty."""
    k0 = (budget_pct * n) // 100
    pts = []
    for i in range(steps + 1):
        kt = (k0 * (steps - i)) // steps
        km = k_mid_for(n, budget_pct, rho, kt)
        pts.append((kt, km))
        if kt + km >= n or kt == 0:
            break
    return pts


def group_error(mats: Sequence[Tuple[ColumnStore, ColumnStore]], xs: Sequence[np.ndarray],
                k_top: int, k_mid: int) -> float:
    """sum over tokens and the group's matrices of ||y_tiered - W x||^2 (fp64)."""
    err = 0.0
    for x in xs:
        F, A = plan_tiers(x, k_top, k_mid)
        n = len(x)
        every = np.arange(n, dtype=np.int32)
        none = np.zeros(0, dtype=np.int32)
        for full, approx in mats:
            y = tiered_product(x, F, A, full, approx)
            d = tiered_product(x, every, none, full, None)
            err += float(((y - d) ** 2).sum())
    return err


def step2_grid(err_of: Callable[[int, int], float], n: int, budget_pct: int, rho: Fraction,
               steps: int):
    """Returns the chosen (k_top, k_mid) and the table [(k_top, k_mid, error)]."""
    table = [(kt, km, err_of(kt, km)) for kt, km in grid_points(n, budget_pct, rho, steps)]
    best = min(range(len(table)), key=lambda i: (table[i][2], i))
    return (table[best][0], table[best][1]), table


def layer_budget(budgets: Sequence[int], dense_bytes: Sequence[int]) -> Fraction:
    """A layer's read budget: the groups' budgets weighted by their dense sizes."""
    return Fraction(sum(b * d for b, d in zip(budgets, dense_bytes)), 100 * sum(dense_bytes))


def step1_greedy(err_of: Sequence[Callable[[int], float]], dense_bytes: Sequence[int],
                 target_pct: int, delta: int = 5):
    """Step 1: every group starts dense (budget 100, k_mid = 0); each round
    lowers by `delta` the group whose reduction raises the layer's error
    least, until the layer budget reaches the target. err_of[g](budget) is
    group g's error at that budget with k_mid = 0. Returns the final budgets
    and the rounds [(group, new budget)]."""
    G = len(err_of)
    b = [100] * G
    cur = [err_of[g](100) for g in range(G)]
    rounds = []
    while layer_budget(b, dense_bytes) > Fraction(target_pct, 100):
        best = None
        for g in range(G):
            if b[g] - delta < 0:
                continue
            e = err_of[g](b[g] - delta)
            rise = e - cur[g]
            if best is None or rise < best[0]:
                best = (rise, g, e)
        if best is None:
            break
        _, g, e = best
        b[g] -= delta
        cur[g] = e
        rounds.append((g, b[g]))
    return b, rounds
