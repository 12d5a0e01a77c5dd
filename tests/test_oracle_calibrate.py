"""Pins for the calibration oracle (SpAx page section 5.2; no GPU): the grid
against a brute-force reading of Eq. 5, closed forms of the two searches."""
from fractions import Fraction

import numpy as np

import oracle as O
import oracle.spax_calibrate as C
import workloads as WL


def _brute_k_mid(n, budget_pct, rho, k_top):
    # the largest k_mid whose bytes fit the budget (Eq. 5), by counting up
    km = 0
    while k_top + km < n and (k_top + (km + 1) * rho) * 100 <= budget_pct * n:
        km += 1
    return km


def test_grid_follows_eq5_and_stops_at_an_empty_tier():
    for n, pct, rho, steps in [(4096, 40, Fraction(264, 1024), 10), (100, 50, Fraction(1, 4), 7),
                               (11008, 35, Fraction(66, 256), 12), (64, 90, Fraction(1, 2), 5),
                               (512, 5, Fraction(1, 8), 4)]:
        pts = C.grid_points(n, pct, rho, steps)
        assert pts[0] == ((pct * n) // 100, _brute_k_mid(n, pct, rho, (pct * n) // 100))
        for i, (kt, km) in enumerate(pts):
            assert km == _brute_k_mid(n, pct, rho, kt)
            assert (kt + km * rho) * 100 <= pct * n
            if i:
                assert kt < pts[i - 1][0] and km >= pts[i - 1][1]
        last = pts[-1]
        assert last[0] + last[1] == n or last[0] == 0
        assert all(kt + km < n and kt > 0 for kt, km in pts[:-1])


def test_group_error_closed_forms():
    Wt = WL.weights_fp16(71, 0, "w", 256, 64, 0.02)
    xs = [WL.laplace_fp16(71, 0, "x", t, 64) for t in range(3)]
    mats = [(O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt))]
    assert C.group_error(mats, xs, 64, 0) == 0.0
    dense = sum(float(((x.astype(np.float64) @ Wt.astype(np.float64)) ** 2).sum()) for x in xs)
    assert np.isclose(C.group_error(mats, xs, 0, 0), dense, rtol=1e-12)


def test_step2_picks_the_largest_k_mid_when_the_middle_tier_is_exact():
    # one magnitude per column: the two-scale sign code rebuilds it exactly,
    # so every column moved from the top tier to the middle tier (and every
    # column added to it) only lowers the error
    rs = np.random.default_rng(72)
    n, R = 96, 128
    Wt = (rs.choice([-1.0, 1.0], (n, R)) * rs.uniform(0.01, 0.05, (n, 1))).astype(np.float16)
    full, approx = O.ColumnStore("fp16", Wt), O.ColumnStore("sign2", Wt)
    assert np.array_equal(approx.columns(np.arange(n)), Wt.astype(np.float64))
    xs = [WL.laplace_fp16(72, 0, "x", t, n) for t in range(2)]
    rho = Fraction(R // 4 + 4, 2 * R)
    (kt, km), table = C.step2_grid(lambda a, b: C.group_error([(full, approx)], xs, a, b),
                                   n, 40, rho, 8)
    assert (kt, km) == table[-1][:2]
    errs = [e for _, _, e in table]
    assert all(b < a for a, b in zip(errs, errs[1:]))


def test_step1_reduces_a_group_that_costs_nothing_first():
    n, R = 64, 128
    Wa = WL.weights_fp16(73, 0, "w", R, n, 0.02)
    Wz = np.zeros((n, R), dtype=np.float16)          # group 1 contributes nothing
    xs = [WL.laplace_fp16(73, 0, "x", t, n) for t in range(2)]
    stores = [[(O.ColumnStore("fp16", W), O.ColumnStore("int4", W))] for W in (Wa, Wz)]
    err_of = [lambda b, s=s: C.group_error(s, xs, (b * n) // 100, 0) for s in stores]
    dense = [R * n * 2, R * n * 2]
    budgets, rounds = C.step1_greedy(err_of, dense, 50)
    assert rounds == [(1, b) for b in range(95, -1, -5)]
    assert budgets == [100, 0]
    assert C.layer_budget(budgets, dense) == Fraction(1, 2)
    # a lower target then lowers group 0 as well; its budget only falls
    budgets2, rounds2 = C.step1_greedy(err_of, dense, 30)
    assert rounds2[:20] == rounds and budgets2 == [60, 0]
    assert [b for g, b in rounds2 if g == 0] == [95, 90, 85, 80, 75, 70, 65, 60]


def test_library_calibration_prices_every_format_like_the_workloads():
    """The library's calibration (Eq. 5's rho) and the workloads' byte
    accounting count a stored column's bytes the same way, for every tier
    format (host logic, no GPU)."""
    import activation_sparse_decode_token_amd as spax
    from activation_sparse_decode_token_amd import calibrate as K
    from workloads.accounting import column_bytes
    names = {spax.FMT_FP16: "fp16", spax.FMT_INT4_G128: "int4", spax.FMT_INT2_G128: "int2",
             spax.FMT_SIGN2: "sign2", spax.FMT_TRELLIS: "trellis"}
    for fmt, name in names.items():
        for rows in (128, 4096, 12288, 28672):
            assert K.column_bytes(fmt, rows) == column_bytes(name, rows), (name, rows)
    assert K.column_bytes(spax.FMT_NONE, 4096) == 0
