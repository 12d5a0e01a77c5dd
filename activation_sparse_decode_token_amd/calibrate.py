"""Offline calibration of the tier sizes (SpAx page, section 5.2) on the GPU.

Eq. 5 gives a group's read budget, (k_top + rho k_mid) / n, with rho the
middle tier's bytes per column over the top tier's. Step 1 starts every
group of a layer dense (budget 1, k_mid = 0) and repeatedly lowers by 0.05
the group whose reduction raises the layer's l2 output error least, until the
layer budget (the groups' budgets weighted by their dense sizes) reaches its
target. Step 2 then lowers k_top in equal steps at the group's budget,
raising k_mid to keep the budget, until a tier runs empty, and keeps the
setting with the smallest error.

Every product runs in the library (spax_plan_tiers, then spax_tiered_gemv);
a token's dense reference is the library's product with every column in the
top tier. The squared errors are summed in fp64 by the library too
(spax_sq_error, one accumulator over the tokens), so one evaluation of a
setting enqueues its tokens' work and synchronises once, to read the sum. Budgets are
integer percentages and Eq. 5 is evaluated in exact integer arithmetic, so
the grid of tier sizes is exact. A group's error is summed over its
calibration tokens and all its stored rows (stacked q, k, v; interleaved
gate and up); groups are evaluated on their own inputs, so a layer's error is
the sum of its groups' errors. Offline tooling: nothing here is on the
per-token path.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple


from . import (FMT_FP16, FMT_INT2_G128, FMT_INT4_G128, FMT_NONE, FMT_SIGN2, FMT_TRELLIS,
               Matrix, gemv_workspace_bytes, plan_tiers, sq_error, tiered_gemv)

__all__ = ["column_bytes", "rho_of", "k_mid_for_budget", "grid", "Group", "step2", "step1",
           "layer_budget"]


def column_bytes(fmt: int, rows: int) -> int:
    """Stored bytes of one column: values, or codes plus their fp16 scales."""
    if fmt == FMT_FP16:
        return 2 * rows
    if fmt == FMT_INT4_G128:
        return rows // 2 + 2 * (rows // 128)
    if fmt == FMT_INT2_G128:
        return rows // 4 + 2 * (rows // 128)
    if fmt == FMT_SIGN2:
        return rows // 4 + 4
    if fmt == FMT_TRELLIS:   # the codebook is shared by every column
        return rows // 4 + 2
    if fmt == FMT_NONE:
        return 0
    raise ValueError(fmt)


def rho_of(W: Matrix) -> Fraction:
    """Middle-tier bytes per column over top-tier bytes per column."""
    return Fraction(column_bytes(W.approx_fmt, W.rows), column_bytes(W.full_fmt, W.rows))


def k_mid_for_budget(n: int, budget_pct: int, rho: Fraction, k_top: int) -> int:
    """The most middle-tier columns that fit beside k_top in the budget."""
    spare = budget_pct * n - 100 * k_top          # 100 x (budget n - k_top)
    if spare <= 0:
        return 0
    return min(n - k_top, (spare * rho.denominator) // (100 * rho.numerator))


def grid(n: int, budget_pct: int, rho: Fraction, steps: int) -> List[Tuple[int, int]]:
    """Step 2's settings: k_top = floor(k0 (steps - i) / steps) from the
    all-top setting k0 = floor(budget n), each with the k_mid that fills the
    budget, up to and including the first setting with an empty tier."""
    k0 = budget_pct * n // 100
    out = []
    for i in range(steps + 1):
        kt = k0 * (steps - i) // steps
        km = k_mid_for_budget(n, budget_pct, rho, kt)
        out.append((kt, km))
        if kt == 0 or kt + km >= n:
            break
    return out


class Group:
    """One ranking group (a stored matrix) with its calibration inputs."""

    def __init__(self, W: Matrix, xs: Sequence, stream=None):
        import torch
        self.W, self.xs, self.stream = W, list(xs), stream
        self.evaluations = 0   # error() calls, for reporting
        dev = self.xs[0].device
        self.n = W.cols
        self.ws = torch.zeros(gemv_workspace_bytes(W), dtype=torch.uint8, device=dev)
        self.F = torch.empty(self.n, dtype=torch.int32, device=dev)
        self.A = torch.empty(self.n, dtype=torch.int32, device=dev)
        self.y = torch.empty(W.rows, dtype=torch.float16, device=dev)
        self.acc = torch.zeros(1, dtype=torch.float64, device=dev)
        self.dense = []
        for x in self.xs:  # the dense references stay on the device
            d = torch.empty(W.rows, dtype=torch.float16, device=dev)
            self._product(x, self.n, 0, d)
            self.dense.append(d)
        torch.cuda.synchronize()

    def _product(self, x, k_top: int, k_mid: int, y) -> None:
        """Enqueues the tiered product of x into y (no synchronisation)."""
        plan_tiers(x, self.n, k_top, k_mid, self.F, self.A, self.stream)
        tiered_gemv(self.W, x, self.F, k_top, self.A, k_mid, y, self.ws, stream=self.stream)

    def dense_bytes(self) -> int:
        return self.n * column_bytes(self.W.full_fmt, self.W.rows)

    def error(self, k_top: int, k_mid: int) -> float:
        """sum over tokens of ||y_tiered - y_dense||^2 over the stored rows:
        every token's product and squared distance on the stream, then one
        synchronisation to read the fp64 sum."""
        import torch
        self.evaluations += 1
        for i, (x, d) in enumerate(zip(self.xs, self.dense)):
            self._product(x, k_top, k_mid, self.y)
            sq_error(self.y, d, self.W.rows, self.acc, accumulate=i > 0, stream=self.stream)
        torch.cuda.synchronize()
        return float(self.acc.cpu()[0])


def step2(g: Group, budget_pct: int, steps: int = 10):
    """Returns the chosen (k_top, k_mid) and the table [(k_top, k_mid, error)]."""
    table = [(kt, km, g.error(kt, km)) for kt, km in grid(g.n, budget_pct, rho_of(g.W), steps)]
    i = min(range(len(table)), key=lambda j: (table[j][2], j))
    return table[i][:2], table


def layer_budget(budgets: Sequence[int], dense: Sequence[int]) -> Fraction:
    return Fraction(sum(b * d for b, d in zip(budgets, dense)), 100 * sum(dense))


def step1(groups: Sequence[Group], target_pct: int, delta: int = 5):
    """Returns the groups' budgets (percent) and the rounds [(group, budget)]."""
    dense = [g.dense_bytes() for g in groups]
    b = [100] * len(groups)
    err = [g.error(g.n, 0) for g in groups]
    rounds = []
    while layer_budget(b, dense) > Fraction(target_pct, 100):
        pick = None
        for i, g in enumerate(groups):
            if b[i] < delta:
                continue
            e = g.error((b[i] - delta) * g.n // 100, 0)
            if pick is None or e - err[i] < pick[0]:
                pick = (e - err[i], i, e)
        if pick is None:
            break
        _, i, e = pick
        b[i] -= delta
        err[i] = e
        rounds.append((i, b[i]))
    return b, rounds
