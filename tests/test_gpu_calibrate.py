"""Offline tier-size calibration on the GPU (SpAx page section 5.2) against
the calibration oracle: the same grids of tier sizes, errors within the fp16
output rounding, the same choices (up to near ties), the same Step 1 rounds."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import oracle.spax_calibrate as C
import workloads as WL
from tests.spax_testlib import log, to_dev

pytestmark = pytest.mark.gpu

HIDDEN, INTER = 512, 1408


def _layer():
    """A small layer's four groups as stored matrices, host copies and inputs."""
    import activation_sparse_decode_token_amd as spax
    from activation_sparse_decode_token_amd.layouts import build_matrix, glu_interleave, stack_rows
    w = {m: WL.weights_fp16(840, 0, m, r, c, 0.02) for m, r, c in
         [("q", HIDDEN, HIDDEN), ("k", HIDDEN, HIDDEN), ("v", HIDDEN, HIDDEN),
          ("o", HIDDEN, HIDDEN), ("gate", INTER, HIDDEN), ("up", INTER, HIDDEN),
          ("down", HIDDEN, INTER)]}
    d = {m: to_dev(v) for m, v in w.items()}
    stored = {
        "qkv": (build_matrix(stack_rows([d["q"], d["k"], d["v"]])),
                np.concatenate([w["q"], w["k"], w["v"]], axis=1)),
        "o": (build_matrix(d["o"]), w["o"]),
        "gu": (build_matrix(glu_interleave(d["gate"], d["up"]),
                            layout=spax.LAYOUT_GLU_INTERLEAVED),
               np.concatenate([w["gate"].reshape(HIDDEN, -1, 1, 128),
                               w["up"].reshape(HIDDEN, -1, 1, 128)], axis=2).reshape(HIDDEN, -1)),
        "down": (build_matrix(d["down"]), w["down"]),
    }
    xs = {g: [WL.laplace_fp16(840, i, "x", t, stored[g][1].shape[0]) for t in range(2)]
          for i, g in enumerate(stored)}
    return stored, xs


@pytest.mark.parametrize("n", [0, 1, 1023, 1025, 57344])
def test_sq_error_kernel(n):
    """spax_sq_error against the fp64 sum of squared differences formed on
    the host (each difference of two fp16 values is exact in fp64; the sums
    differ only in their order); accumulate mode adds to the stored value;
    two calls give the same bits."""
    import torch
    import activation_sparse_decode_token_amd as spax
    rs = np.random.default_rng(850 + n)
    y = rs.standard_normal(n).astype(np.float16)
    r = (y.astype(np.float32) + 0.01 * rs.standard_normal(n)).astype(np.float16)
    r[: n // 7] = y[: n // 7]  # some equal pairs
    want = float(((y.astype(np.float64) - r.astype(np.float64)) ** 2).sum())
    acc = torch.full((1,), 123.5, dtype=torch.float64, device="cuda:0")
    yd, rd = to_dev(y), to_dev(r)
    spax.sq_error(yd, rd, n, acc)
    torch.cuda.synchronize()
    got = float(acc.cpu()[0])
    assert abs(got - want) <= 1e-12 * want + 1e-300, (got, want)
    spax.sq_error(yd, rd, n, acc, accumulate=True)
    torch.cuda.synchronize()
    assert float(acc.cpu()[0]) == got + got
    spax.sq_error(yd, rd, n, acc)
    torch.cuda.synchronize()
    assert float(acc.cpu()[0]) == got  # the same bits again
    log(f"sq_error n={n}: {got:.6g} (host {want:.6g})")


def test_step2_grid_matches_the_oracle():
    import activation_sparse_decode_token_amd.calibrate as K
    stored, xs = _layer()
    for g, (W, Wt) in stored.items():
        grp = K.Group(W, [to_dev(x) for x in xs[g]])
        mats = [(O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt))]
        rho = Fraction(W.rows // 2 + 2 * (W.rows // 128), 2 * W.rows)
        assert K.rho_of(W) == rho
        (kt, km), table = K.step2(grp, 40, 6)
        (okt, okm), otable = C.step2_grid(lambda a, b: C.group_error(mats, xs[g], a, b),
                                          grp.n, 40, rho, 6)
        assert [r[:2] for r in table] == [r[:2] for r in otable], g
        for (_, _, e), (_, _, oe) in zip(table, otable):
            assert abs(e - oe) <= 1e-2 * oe + 1e-9, (g, e, oe)
        oerr = {r[:2]: r[2] for r in otable}
        assert oerr[(kt, km)] <= min(oerr.values()) * (1 + 1e-2), g
        log(f"step 2 {g}: GPU picks ({kt}, {km}), oracle ({okt}, {okm})")



def test_step2_with_the_trellis_tier():
    """Step 2 on a group whose middle tier is trellis-coded: rho from the
    trellis column bytes (codes plus one fp16 scale), the library's errors
    against the oracle's, which rebuilds the same codes itself."""
    import activation_sparse_decode_token_amd as spax
    import activation_sparse_decode_token_amd.calibrate as K
    from activation_sparse_decode_token_amd.layouts import build_matrix
    from tests.spax_testlib import TrellisStore, to_host
    R, n = 512, 512
    Wt = WL.weights_fp16(841, 0, "w", R, n, 0.02)
    cb = WL.trellis_codebook(1)
    W = build_matrix(to_dev(Wt), spax.FMT_FP16, spax.FMT_TRELLIS, codebook=to_dev(cb))
    st = TrellisStore(to_host(W._keep[2]), to_host(W._keep[3]), cb)
    xs = [WL.laplace_fp16(841, t, "x", n, n) for t in range(2)]
    grp = K.Group(W, [to_dev(x) for x in xs])
    rho = Fraction(R // 4 + 2, 2 * R)
    assert K.rho_of(W) == rho
    (kt, km), table = K.step2(grp, 40, 6)
    mats = [(O.ColumnStore("fp16", Wt), st)]
    (okt, okm), otable = C.step2_grid(lambda a, b: C.group_error(mats, xs, a, b), n, 40, rho, 6)
    assert [r[:2] for r in table] == [r[:2] for r in otable]
    for (_, _, e), (_, _, oe) in zip(table, otable):
        assert abs(e - oe) <= 1e-2 * oe + 1e-9, (e, oe)
    oerr = {r[:2]: r[2] for r in otable}
    assert oerr[(kt, km)] <= min(oerr.values()) * (1 + 1e-2)
    log(f"step 2 trellis: GPU picks ({kt}, {km}), oracle ({okt}, {okm})")

def test_step1_rounds_match_the_oracle():
    import activation_sparse_decode_token_amd.calibrate as K
    stored, xs = _layer()
    names = list(stored)
    groups = [K.Group(stored[g][0], [to_dev(x) for x in xs[g]]) for g in names]
    budgets, rounds = K.step1(groups, 70)
    mats = [[(O.ColumnStore("fp16", stored[g][1]), O.ColumnStore("int4", stored[g][1]))]
            for g in names]
    err_of = [lambda b, i=i: C.group_error(mats[i], xs[names[i]], b * groups[i].n // 100, 0)
              for i in range(len(names))]
    dense = [gr.dense_bytes() for gr in groups]
    obudgets, orounds = C.step1_greedy(err_of, dense, 70)
    assert C.layer_budget(budgets, dense) <= Fraction(70, 100)
    if rounds != orounds:
        # the searches may part only at a near tie: at the first differing
        # round, both choices raise the oracle's error by nearly the same amount
        r = next(i for i, (a, b) in enumerate(zip(rounds, orounds)) if a != b)
        b = [100] * len(names)
        for g, nb in orounds[:r]:
            b[g] = nb
        rise = lambda g: err_of[g](b[g] - 5) - err_of[g](b[g])
        ga, go = rounds[r][0], orounds[r][0]
        assert abs(rise(ga) - rise(go)) <= 1e-2 * max(rise(ga), rise(go)), (r, ga, go)
    log(f"step 1: budgets {dict(zip(names, budgets))} in {len(rounds)} rounds")
