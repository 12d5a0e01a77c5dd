"""Pins for the CPU oracle (no GPU).

Every check here ties the oracle to something other than itself: values the
pages print or that follow from their worked examples (tests/golden/, each
file citing its passage), closed forms, exact rational arithmetic, brute
force over tiny inputs, and invariants that any correct result satisfies.
"""
import itertools
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as WL
from workloads import accounting as ACC


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fp16 rounding

def _exact_fp16_rne(v: float) -> float:
    """Round a double to the fp16 grid exactly (rational arithmetic)."""
    if v == 0 or math.isnan(v) or math.isinf(v):
        return v
    sign = -1.0 if v < 0 else 1.0
    a = Fraction(abs(v))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val > 65504:
        return sign * math.inf
    return sign * float(val)


def test_fp16_round_matches_exact_rational_rounding():
    rs = random.Random(1)
    vals = []
    for _ in range(4000):
        e = rs.uniform(-27, 16.5)
        vals.append(rs.choice([-1, 1]) * 2.0 ** e)
    # exact midpoints between neighbouring fp16 values, and one double either side
    all16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    pick = rs.sample(range(len(all16) - 1), 1500)
    for i in pick:
        mid = (all16[i] + all16[i + 1]) / 2
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, 1e9), -mid]
    vals += [65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26,
             3 * 2.0 ** -26, 1e-9, 0.1, 1 / 3]
    got = O.fp16_round(np.array(vals)).astype(np.float64)
    want = np.array([_exact_fp16_rne(v) for v in vals])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- tier selection

def test_magnitude_key_orders_like_abs():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    finite = np.isfinite(x)
    xs = x[finite]
    key = O.magnitude_key(xs)
    a = np.abs(xs.astype(np.float64))
    # key order agrees with |x| order (equal keys <=> equal magnitudes)
    o1 = np.argsort(key, kind="stable")
    assert np.all(np.diff(a[o1]) >= 0)
    assert np.array_equal(key[xs == 0], np.zeros(np.count_nonzero(xs == 0), dtype=np.int64))
    inf_key = O.magnitude_key(np.array([np.inf, -np.inf], dtype=np.float16))
    assert np.all(inf_key > key.max())


def _brute_plan(x, kf, ka):
    """Definition-level selection: a valid top-k set has every member at least
    as large in |x| as every non-member; among valid sets the one with the
    smallest index sum wins (lower index ranks first on ties)."""
    mags = [abs(float(v)) for v in x]

    def best(cands, k):
        cands = list(cands)
        found = None
        for S in itertools.combinations(cands, k):
            rest = [i for i in cands if i not in S]
            if S and rest and min(mags[i] for i in S) < max(mags[i] for i in rest):
                continue
            if found is None or sum(S) < sum(found):
                found = S
        return sorted(found)

    F = best(range(len(x)), kf)
    A = best([i for i in range(len(x)) if i not in F], ka)
    return F, A


def _check_against_brute(x):
    n = len(x)
    for kf in range(n + 1):
        for ka in range(n - kf + 1):
            F, A = O.plan_tiers(x, kf, ka)
            bF, bA = _brute_plan(x, kf, ka)
            assert list(F) == bF and list(A) == bA, (x, kf, ka)


def test_plan_brute_force_exhaustive_small_alphabet():
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 0.5], dtype=np.float16)
    for n in range(1, 5):
        for combo in itertools.product(range(len(alphabet)), repeat=n):
            _check_against_brute(alphabet[list(combo)])


def test_plan_brute_force_random_n5_n7():
    rs = np.random.default_rng(7)
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, 3.0], dtype=np.float16)
    for n in (5, 6, 7):
        for _ in range(60):
            _check_against_brute(alphabet[rs.integers(0, len(alphabet), n)])


def test_plan_maximises_kept_energy():
    """SpAx page section 2: top-k keeps the entries that minimise the energy
    of the dropped ones, sum_{dropped} x_i^2. Check F and F u A reach the
    maximum kept energy over all subsets of their size (brute force)."""
    rs = np.random.default_rng(3)
    for _ in range(40):
        n = int(rs.integers(4, 11))
        x = (rs.integers(-4, 5, n) / 2.0).astype(np.float16)
        e = x.astype(np.float64) ** 2
        kf = int(rs.integers(0, n + 1))
        ka = int(rs.integers(0, n - kf + 1))
        F, A = O.plan_tiers(x, kf, ka)
        best_f = max(sum(e[list(S)]) for S in itertools.combinations(range(n), kf))
        best_fa = max(sum(e[list(S)]) for S in itertools.combinations(range(n), kf + ka))
        assert e[F].sum() == best_f
        assert e[np.concatenate([F, A]).astype(int)].sum() == best_fa


def test_fig2_worked_example(golden_dir):
    g = _load(golden_dir, "fig2_three_tier.json")
    x = np.array(g["x"], dtype=np.float16)
    F, A = O.plan_tiers(x, g["k_top"], g["k_mid"])
    assert list(F) == g["expected_full"]
    assert list(A) == g["expected_approx"]
    skip = sorted(set(range(g["n"])) - set(F) - set(A))
    assert skip == g["expected_skip"]
    R = g["rows"]
    Wt = np.zeros((g["n"], R), dtype=np.float16)
    Wt[:, :4] = np.array(g["columns_first4"], dtype=np.float16)
    full = O.ColumnStore("fp16", Wt)
    approx = O.ColumnStore("int4", Wt)
    c0 = approx.columns([0])[0]
    c3 = approx.columns([3])[0]
    assert list(c0[:4]) == g["C0hat_first4"] and not np.any(c0[4:])
    assert list(c3[:4]) == g["C3hat_first4"] and not np.any(c3[4:])
    assert float(approx.scales[0, 0]) == g["C0_scale"]
    assert float(approx.scales[3, 0]) == g["C3_scale"]
    y = O.tiered_product(x, F, A, full, approx)
    assert list(y[:4]) == g["expected_y_first4"]
    assert not np.any(y[4:])


def test_plan_invariants_on_config_inputs():
    for cfg, n, split in [(1, 1024, WL.CONFIGS[1].splits[0]),
                          (2, 4096, WL.CONFIGS[2].splits[0]),
                          (3, 11008, WL.CONFIGS[3].splits[2]),
                          (5, 28672, WL.CONFIGS[5].splits[0])]:
        x = WL.laplace_fp16(cfg, 0, "x", 0, n)
        kf, ka = WL.tier_counts(n, split)
        F, A = O.plan_tiers(x, kf, ka)
        assert len(F) == kf and len(A) == ka
        assert np.all(np.diff(F) > 0) and np.all(np.diff(A) > 0)
        assert not set(F) & set(A)
        key = np.abs(x.astype(np.float64))
        S = np.setdiff1d(np.arange(n), np.concatenate([F, A]))
        if kf and ka:
            assert key[F].min() >= key[A].max()
        if ka and len(S):
            assert key[A].min() >= key[S].max()
        # ties across a boundary: the higher tier holds the lower indices
        for hi, lo in ((F, A), (A, S), (F, S)):
            if len(hi) and len(lo):
                t = key[hi].min()
                if key[lo].max() == t:
                    assert hi[key[hi] == t].max() < lo[key[lo] == t].min()


def test_tier_counts_match_stated_sizes():
    # (n, split) -> (k_full, k_approx) as listed for the five workloads
    cases = {
        (1024, (50, 25, 25)): (256, 256),
        (4096, (40, 30, 30)): (1229, 1229),
        (4096, (30, 20, 50)): (2048, 819),
        (11008, (30, 20, 50)): (5504, 2202),
        (11008, (70, 20, 10)): (1101, 2201),
        (8192, (50, 30, 20)): (1638, 2458),
        (28672, (50, 30, 20)): (5734, 8602),
        (4096, (50, 25, 25)): (1024, 1024),
        (11008, (50, 25, 25)): (2752, 2752),
    }
    for (n, sp), want in cases.items():
        assert WL.tier_counts(n, WL.TierSplit(*sp)) == want


def test_plan_special_cases():
    rs = np.random.default_rng(0)
    x = rs.laplace(size=300).astype(np.float16)
    F, A = O.plan_tiers(x, 300, 0)
    assert np.array_equal(F, np.arange(300)) and len(A) == 0
    F, A = O.plan_tiers(x, 0, 0)
    assert len(F) == 0 and len(A) == 0
    F, A = O.plan_tiers(x, 0, 300)
    assert len(F) == 0 and np.array_equal(A, np.arange(300))
    same = np.full(50, -1.5, dtype=np.float16)
    F, A = O.plan_tiers(same, 7, 11)
    assert np.array_equal(F, np.arange(7)) and np.array_equal(A, np.arange(7, 18))
    # exact scaling by a power of two keeps the ranking
    y = rs.uniform(0.5, 4, 200).astype(np.float16) * rs.choice([-1, 1], 200).astype(np.float16)
    for e in (-3, 2):
        F1, A1 = O.plan_tiers(y, 40, 60)
        F2, A2 = O.plan_tiers((y.astype(np.float64) * 2.0 ** e).astype(np.float16), 40, 60)
        assert np.array_equal(F1, F2) and np.array_equal(A1, A2)
    # +0 and -0 tie: the lower index wins
    z = np.array([-0.0, 0.0, -0.0, 1.0], dtype=np.float16)
    F, A = O.plan_tiers(z, 2, 1)
    assert list(F) == [0, 3] and list(A) == [1]
    with pytest.raises(ValueError):
        O.plan_tiers(z, 3, 2)


# ---------------------------------------------------------------- packing

def test_int4_golden(golden_dir):
    g = _load(golden_dir, "int4_pack_example.json")
    col = np.zeros(128, dtype=np.float16)
    col[:8] = g["group_first8"]
    codes, scales = O.pack_int4_g128(col[None, :])
    assert float(scales[0, 0]) == g["expected_scale"]
    assert list(codes[0, :4]) == g["expected_bytes_first4"]
    assert np.all(codes[0, 4:] == g["expected_bytes_rest"])
    what = O.dequant_int4_g128(codes, scales)[0]
    assert list(what[:8]) == [q * g["expected_scale"] for q in g["expected_q_first8"]]


def test_int2_golden(golden_dir):
    g = _load(golden_dir, "int2_pack_example.json")
    col = np.zeros(128, dtype=np.float16)
    col[:8] = g["group_first8"]
    codes, scales = O.pack_int2_g128(col[None, :])
    assert float(scales[0, 0]) == g["expected_scale"]
    assert list(codes[0, :2]) == g["expected_bytes_first2"]
    assert np.all(codes[0, 2:] == g["expected_bytes_rest"])
    what = O.dequant_int2_g128(codes, scales)[0]
    assert list(what[:8]) == g["expected_what_first8"]


@pytest.mark.parametrize("fmt", ["int4", "int2"])
def test_pack_error_bound_and_layout(fmt):
    pack = O.pack_int4_g128 if fmt == "int4" else O.pack_int2_g128
    deq = O.dequant_int4_g128 if fmt == "int4" else O.dequant_int2_g128
    Wt = WL.weights_fp16(99, 0, "w", 512, 64, 0.02)
    codes, scales = pack(Wt)
    n, R = Wt.shape
    assert codes.shape == (n, R // (2 if fmt == "int4" else 4)) and codes.dtype == np.uint8
    assert scales.shape == (n, R // 128) and scales.dtype == np.float16
    w = Wt.astype(np.float64)
    what = deq(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(w - what) <= s / 2)
    # the scale is the group maximum over the top level (7 or 1.5), one fp16 rounding
    m = np.abs(w).reshape(n, R // 128, 128).max(axis=2)
    top = 7.0 if fmt == "int4" else 1.5
    assert np.all(np.abs(scales.astype(np.float64) - m / top) <= np.abs(m / top) * 2.0 ** -11)
    # round trip: re-packing the reconstruction gives the same codes and scales
    c2, s2 = pack(what.astype(np.float16))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_pack_on_grid_and_zero_groups():
    rs = np.random.default_rng(5)
    s = 2.0 ** -6
    q = rs.integers(-7, 8, (3, 256))
    q[:, 0] = 7
    q[:, 128] = -7
    Wt = (q * s).astype(np.float16)
    codes, scales = O.pack_int4_g128(Wt)
    assert np.all(scales == np.float16(s))
    assert np.array_equal(O.dequant_int4_g128(codes, scales), q * s)
    zero = np.zeros((2, 256), dtype=np.float16)
    c4, s4 = O.pack_int4_g128(zero)
    c2, s2 = O.pack_int2_g128(zero)
    assert not np.any(c4) and not np.any(s4.astype(np.float64))
    assert np.all(c2 == 0xAA) and not np.any(s2.astype(np.float64))
    assert not np.any(O.dequant_int2_g128(c2, s2))


# ---------------------------------------------------------------- two-scale sign code

def _sign2_levels(s0: Fraction, s1: Fraction):
    # code order u = 0..3: (+,+), (+,-), (-,+), (-,-)  (SpAx page section 5.1, Eq. 4)
    return [s0 + s1, s0 - s1, -s0 + s1, -s0 - s1]


def _sign2_brute(col: np.ndarray):
    """Eq. 4 by exact rational arithmetic: greedy scales from exact means,
    rounded by the rational fp16 rounding; each code the smallest u among
    the exact minimisers of (w - a s0 - b s1)^2."""
    w = [Fraction(float(v)) for v in col.astype(np.float64)]
    R = len(w)
    s0 = Fraction(_exact_fp16_rne(float(sum(abs(v) for v in w) / R)))
    e1 = [1 if v >= 0 else -1 for v in w]
    s1 = Fraction(_exact_fp16_rne(float(sum(abs(v - e * s0) for v, e in zip(w, e1)) / R)))
    L = _sign2_levels(s0, s1)
    u = []
    for v in w:
        d = [(v - lv) ** 2 for lv in L]
        u.append(min(range(4), key=lambda k: (d[k], k)))
    return s0, s1, u


def test_sign2_golden(golden_dir):
    g = _load(golden_dir, "sign2_pack_example.json")
    col = np.tile(np.array(g["pattern"], dtype=np.float16), g["rows"] // 4)
    codes, scales = O.pack_sign2(col[None, :])
    assert float(scales[0, 0]) == g["expected_s0"] and float(scales[0, 1]) == g["expected_s1"]
    assert np.all(codes[0] == g["expected_byte"])
    what = O.dequant_sign2(codes, scales)[0]
    assert list(what[:4]) == g["expected_what_pattern"]
    u = [(int(codes[0, 0]) >> (2 * r)) & 3 for r in range(4)]
    assert u == g["expected_u_pattern"]


def test_sign2_matches_exact_rational_fit_and_argmin():
    rs = np.random.default_rng(11)
    cols = [WL.weights_fp16(93, 0, "w", 128, 3, 0.02)[c] for c in range(3)]
    # coarse grids force exact ties between levels (midpoints)
    cols.append((rs.integers(-8, 9, 128) * 0.125).astype(np.float16))
    cols.append((rs.integers(-3, 4, 128) * 0.25).astype(np.float16))
    # tiny (subnormal fp16) weights and a lone outlier
    tiny = (rs.integers(-20, 21, 128) * 2.0 ** -24).astype(np.float16)
    cols.append(tiny)
    out = np.zeros(128, dtype=np.float16)
    out[5] = 3.0
    cols.append(out)
    for col in cols:
        codes, scales = O.pack_sign2(col[None, :])
        s0, s1, u = _sign2_brute(col)
        assert Fraction(float(scales[0, 0])) == s0 and Fraction(float(scales[0, 1])) == s1
        got = [(int(codes[0, i // 4]) >> (2 * (i % 4))) & 3 for i in range(128)]
        assert got == u
        what = O.dequant_sign2(codes, scales)[0]
        L = _sign2_levels(s0, s1)
        assert [Fraction(float(v)) for v in what] == [L[k] for k in u]


def test_sign2_closed_forms():
    rs = np.random.default_rng(12)
    # one magnitude: s0 = that magnitude, s1 = 0, exact reconstruction
    c = (rs.choice([-1.0, 1.0], 256) * 0.375).astype(np.float16)
    codes, scales = O.pack_sign2(c[None, :])
    assert float(scales[0, 0]) == 0.375 and float(scales[0, 1]) == 0.0
    assert np.array_equal(O.dequant_sign2(codes, scales)[0], c.astype(np.float64))
    # two magnitudes a > b in equal numbers: s0 = (a + b) / 2, s1 = (a - b) / 2,
    # and the four levels +-a, +-b reproduce every weight exactly
    mags = np.repeat([0.75, 0.25], 128)
    rs.shuffle(mags)
    c = (rs.choice([-1.0, 1.0], 256) * mags).astype(np.float16)
    codes, scales = O.pack_sign2(c[None, :])
    assert float(scales[0, 0]) == 0.5 and float(scales[0, 1]) == 0.25
    assert np.array_equal(O.dequant_sign2(codes, scales)[0], c.astype(np.float64))
    # zero column: both scales 0, code 0, reconstruction 0
    codes, scales = O.pack_sign2(np.zeros((2, 128), dtype=np.float16))
    assert not np.any(codes) and not np.any(scales.astype(np.float64))
    assert not np.any(O.dequant_sign2(codes, scales))
    # negating a column flips every code's signs and keeps the scales
    c = WL.weights_fp16(92, 0, "w", 256, 4, 0.02)
    nz = c[:, :]
    c1, s1 = O.pack_sign2(nz)
    c2, s2 = O.pack_sign2(-nz)
    assert np.array_equal(s1, s2)
    w1 = O.dequant_sign2(c1, s1)
    w2 = O.dequant_sign2(c2, s2)
    # exact ties may resolve differently; the errors are equal everywhere
    assert np.array_equal(np.abs(nz.astype(np.float64) - w1),
                          np.abs(-nz.astype(np.float64) - w2))


def test_sign2_error_bounds_and_layout():
    Wt = WL.weights_fp16(91, 0, "w", 512, 64, 0.02)
    codes, scales = O.pack_sign2(Wt)
    n, R = Wt.shape
    assert codes.shape == (n, R // 4) and codes.dtype == np.uint8
    assert scales.shape == (n, 2) and scales.dtype == np.float16
    w = Wt.astype(np.float64)
    what = O.dequant_sign2(codes, scales)
    s0 = scales[:, 0:1].astype(np.float64)
    s1 = scales[:, 1:2].astype(np.float64)
    # the argmin is never worse than the greedy sign pair, nor than the
    # one-scale sign code alone
    e1 = np.where(w >= 0, 1.0, -1.0)
    e2 = np.where(w - e1 * s0 >= 0, 1.0, -1.0)
    err = np.abs(w - what)
    assert np.all(err <= np.abs(w - (e1 * s0 + e2 * s1)))
    assert np.all(err <= np.abs(w - e1 * s0) + s1)
    # and on N(0, 0.02) weights it removes most of the energy
    assert (err ** 2).sum() < 0.15 * (w ** 2).sum()


# ---------------------------------------------------------------- tiered product

def _fsum_product(x, Wt, idx):
    """Exactly rounded sum of exact products (math.fsum), row by row."""
    R = Wt.shape[1]
    xs = [float(v) for v in x]
    cols = Wt.astype(np.float64)
    return np.array([math.fsum(xs[j] * float(cols[j, i]) for j in idx) for i in range(R)])


def test_all_full_equals_dense_product():
    Wt = WL.weights_fp16(98, 0, "w", 128, 40, 0.02)
    x = WL.laplace_fp16(98, 0, "x", 0, 40)
    full = O.ColumnStore("fp16", Wt)
    F, A = O.plan_tiers(x, 40, 0)
    r = O.tiered_product(x, F, A, full, None)
    want = _fsum_product(x, Wt, range(40))
    assert np.allclose(r, want, rtol=1e-12, atol=1e-15)


def test_all_approx_equals_dense_product_of_reconstruction():
    Wt = WL.weights_fp16(97, 0, "w", 256, 30, 0.02)
    x = WL.laplace_fp16(97, 0, "x", 0, 30)
    for fmt in ("int4", "int2", "sign2"):
        approx = O.ColumnStore(fmt, Wt)
        rec = approx.columns(np.arange(30))
        F, A = O.plan_tiers(x, 0, 30)
        r = O.tiered_product(x, F, A, O.ColumnStore("fp16", Wt), approx)
        want = _fsum_product(x, rec, range(30))
        assert np.allclose(r, want, rtol=1e-12, atol=1e-15)


def test_all_skip_is_exact_zero_and_linearity():
    Wt = WL.weights_fp16(96, 0, "w", 256, 64, 0.02)
    x = WL.laplace_fp16(96, 0, "x", 0, 64)
    full, approx = O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt)
    F, A = O.plan_tiers(x, 0, 0)
    r = O.tiered_product(x, F, A, full, approx)
    assert np.all(r == 0) and not np.any(np.signbit(r))
    F, A = O.plan_tiers(x, 20, 25)
    both = O.tiered_product(x, F, A, full, approx)
    only_f = O.tiered_product(x, F, A[:0], full, approx)
    only_a = O.tiered_product(x, F[:0], A, full, approx)
    assert np.allclose(both, only_f + only_a, rtol=1e-13, atol=1e-16)


def test_eq1_masked_projection():
    """SpAx page section 2 Eq. 1: W (m . x) = sum over kept i of x_i W[:, i]."""
    Wt = WL.weights_fp16(95, 0, "w", 128, 50, 0.02)
    x = WL.laplace_fp16(95, 0, "x", 0, 50)
    F, _ = O.plan_tiers(x, 17, 0)
    mask = np.zeros(50)
    mask[F] = 1
    xm = x.astype(np.float64) * mask
    masked = np.array([math.fsum(xm[j] * float(Wt[j, i]) for j in range(50)) for i in range(128)])
    r = O.tiered_product(x, F, F[:0], O.ColumnStore("fp16", Wt), None)
    assert np.allclose(r, masked, rtol=1e-12, atol=1e-15)


def test_one_hot_columns_closed_form():
    R = 128
    Wt = np.eye(R, dtype=np.float16)
    x = WL.laplace_fp16(94, 0, "x", 0, R)
    F, A = O.plan_tiers(x, 30, 40)
    r = O.tiered_product(x, F, A, O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt))
    want = np.zeros(R)
    want[F] = x[F].astype(np.float64)
    # a one-hot column has m = 1, s = fp16(1/7) = 1170 * 2^-13, q = 7
    want[A] = x[A].astype(np.float64) * 7 * (1170 * 2.0 ** -13)
    assert np.array_equal(r, want)
    r2 = O.tiered_product(x, F, A, O.ColumnStore("fp16", Wt), O.ColumnStore("int2", Wt))
    # int2: s = fp16(1/1.5) = 1365 * 2^-11; the one is coded u = rint(1/s + 1.5) = 3
    # (1.5 s) and every zero u = rint(1.5) = 2 (+0.5 s): the mid-rise code has no zero
    s2 = 1365 * 2.0 ** -11
    want2 = np.zeros(R)
    want2[F] = x[F].astype(np.float64)
    want2 += 0.5 * s2 * x[A].astype(np.float64).sum()
    want2[A] += x[A].astype(np.float64) * s2
    assert np.allclose(r2, want2, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- SwiGLU

def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([1.0]))[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    z = np.linspace(-30, 30, 241)
    # silu(z) - silu(-z) = z, since sigma(z) + sigma(-z) = 1
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-13)
    assert O.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-15)
    assert abs(O.silu(np.array([-60.0]))[0]) < 1e-24
    g = np.array([0.0, 1.0, -2.0, 4.0], dtype=np.float16)
    u = np.array([3.0, 2.0, 1.0, -0.5], dtype=np.float16)
    a = O.swiglu_fp16(g, u)
    want = [0.0, 2 / (1 + math.exp(-1)), -2 / (1 + math.exp(2)), -0.5 * 4 / (1 + math.exp(-4))]
    assert np.array_equal(a, np.array(want).astype(np.float16))


def test_layer_step_groups_share_rankings_and_chain():
    """Section 5.2 / 5.3: q, k, v share one ranking of h; gate and up share
    one of x; down ranks a = silu(g) * u."""
    R, n = 256, 128
    Wq = WL.weights_fp16(93, 0, "q", R, n, 0.02)
    mats = {name: (O.ColumnStore("fp16", Wq), O.ColumnStore("int4", Wq)) for name in "qkv"}
    mats["o"] = mats["q"]
    Wg = WL.weights_fp16(93, 0, "gate", 384, n, 0.02)
    Wu = WL.weights_fp16(93, 0, "up", 384, n, 0.02)
    Wd = WL.weights_fp16(93, 0, "down", n, 384, 0.02)
    mats["gate"] = (O.ColumnStore("fp16", Wg), O.ColumnStore("int4", Wg))
    mats["up"] = (O.ColumnStore("fp16", Wu), O.ColumnStore("int4", Wu))
    mats["down"] = (O.ColumnStore("fp16", Wd), O.ColumnStore("int4", Wd))
    h = WL.laplace_fp16(93, 0, "h", 0, n)
    x = WL.laplace_fp16(93, 0, "x", 0, n)
    ks = {"qkv": (30, 40), "o": (30, 40), "ffn": (40, 30), "down": (100, 100)}
    out = O.layer_step(mats, ks, h=h, z=h, x=x)
    assert np.array_equal(out["q"], out["k"]) and np.array_equal(out["k"], out["v"])
    assert np.array_equal(out["o"], out["q"])
    assert np.array_equal(out["a"], O.swiglu_fp16(out["g"], out["u"]))
    F, A = O.plan_tiers(out["a"], 100, 100)
    assert np.array_equal(F, out["down_lists"][0]) and np.array_equal(A, out["down_lists"][1])


# ---------------------------------------------------------------- accounting

def test_budget_arithmetic_matches_table3(golden_dir):
    g = _load(golden_dir, "table3_budget.json")
    assert round(100 * g["spax_trellis_10pct_gb"] / g["dense_bf16_gb"]) == g["budget_spax_pct"]
    assert round(100 * g["teal_10pct_gb"] / g["dense_bf16_gb"]) == g["budget_teal_pct"]
    # Eq. 5 with our byte counting: bytes touched / dense bytes == budget
    R, n, kf, ka = 4096, 4096, 1229, 1229
    touched = kf * ACC.column_bytes("fp16", R) + ka * ACC.column_bytes("int4", R)
    dense = n * ACC.column_bytes("fp16", R)
    b = ACC.budget(kf, ka, n, ACC.rho("fp16", "int4", R))
    assert touched / dense == pytest.approx(b, rel=1e-15)
    assert ACC.rho("fp16", "int4", R) == 33 / 128
    # per-projection algorithmic bytes for the 4096x4096 40/30/30 case
    assert ACC.gemv_algorithmic_bytes(R, n, kf, ka, "fp16", "int4") == 12_689_832


def test_roofline_helpers_match_lazyweights_example(golden_dir):
    g = _load(golden_dir, "lazyweights_roofline.json")
    tol = g["tolerance_rel"]
    fixed_gb = g["weights_gb_coded"] * g["bits_fixed"] / g["bits_coded"]
    assert fixed_gb == pytest.approx(g["expected_fixed_gb"], rel=tol)
    bw = g["bandwidth_gb_s"] * 1e9
    assert ACC.floor_seconds(fixed_gb * 1e9, bw) * 1e3 == pytest.approx(g["expected_floor_fixed_ms"], rel=tol)
    assert ACC.floor_seconds(g["weights_gb_coded"] * 1e9, bw) * 1e3 == pytest.approx(
        g["expected_floor_coded_ms"], rel=tol)
    lo, hi = g["decode_rate_range_gweights_s"]
    rate = ACC.decode_rate(bw, g["bits_coded"]) / 1e9
    assert lo <= rate <= hi


def test_oracle_is_independent_of_the_library():
    here = os.path.dirname(O.__file__)
    for fn in os.listdir(here):
        if fn.endswith(".py"):
            src = open(os.path.join(here, fn)).read()
            assert "activation_sparse_decode_token_amd" not in src
            assert "ctypes" not in src and "libspax" not in src
