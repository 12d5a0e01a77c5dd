"""The layer kernel's work schedule (spax_layer_schedule, host code, no GPU).

Each group runs on a range of workgroups (gate/up and down on all of them,
q/k/v and o on two disjoint ranges in proportion to their bytes); the
group's units (one per selected column per row tile) are cut into one run
per workgroup of its range. The schedule must partition every tile's
full-tier and approx-tier lists exactly among the workgroups that meet the
tile, name those workgroups consistently (they count arrivals on the tile
and the last adds the partial sums in workgroup order), keep the
partial-sum slots t + i (i: the workgroup's index in the group's range)
distinct, visit the groups in processing order and balance the bytes."""
import numpy as np
import pytest

import activation_sparse_decode_token_amd as spax

P = 0x10000
TILE = 512
ORDER = [spax.GROUP_GATE_UP, spax.GROUP_QKV, spax.GROUP_O, spax.GROUP_DOWN]


def _tile_bytes(fmt):
    return {spax.FMT_FP16: 2 * TILE, spax.FMT_INT4_G128: TILE // 2 + 8,
            spax.FMT_INT2_G128: TILE // 4 + 8, spax.FMT_SIGN2: TILE // 4 + 4,
            spax.FMT_NONE: 0}[fmt]


def _m(rows, cols, ff, af, layout=spax.LAYOUT_PLAIN):
    return spax.Matrix.make(rows, cols, ff, af, P, P if ff == spax.FMT_INT4_G128 else None,
                            P if af else None, P if af else None, spax.RES_DEVICE, layout)


def _layer(hidden, inter, ks, ff=spax.FMT_FP16, af=spax.FMT_INT4_G128, groups=(1, 1, 1, 1)):
    G = spax.LAYOUT_GLU_INTERLEAVED
    mats = [_m(3 * hidden, hidden, ff, af), _m(hidden, hidden, ff, af),
            _m(2 * inter, hidden, ff, af, G), _m(hidden, inter, ff, af)]
    mats = [m if on else None for m, on in zip(mats, groups)]
    return spax.Layer.make(mats, [k[0] for k in ks], [k[1] for k in ks])


LAYERS = {
    # 7B-shaped layer, 50/25/25
    "7b": (4096, 11008, [(1024, 1024), (1024, 1024), (1024, 1024), (2752, 2752)],
           spax.FMT_FP16, spax.FMT_INT4_G128, (1, 1, 1, 1)),
    # 70B-shaped FFN, fp16 full + int2 approx, 50/30/20 (code-only layers,
    # with an int4 full tier, run the per-group launches)
    "70b_ffn": (8192, 28672, [(0, 0), (0, 0), (1638, 2458), (5734, 8602)],
                spax.FMT_FP16, spax.FMT_INT2_G128, (0, 0, 1, 1)),
    # ragged tiles, an empty group and a one-column tier
    "ragged": (640, 1408, [(1, 0), (0, 0), (300, 17), (0, 1)],
               spax.FMT_FP16, spax.FMT_SIGN2, (1, 1, 1, 1)),
    # attention only
    "attn": (4096, 0, [(1229, 1229), (1229, 1229), (0, 0), (0, 0)],
             spax.FMT_FP16, spax.FMT_INT4_G128, (1, 1, 0, 0)),
}


def _rows(hidden, inter):
    return {spax.GROUP_QKV: 3 * hidden, spax.GROUP_O: hidden,
            spax.GROUP_GATE_UP: 2 * inter, spax.GROUP_DOWN: hidden}


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("wgs", [1, 2, 7, 37, 256])
def test_schedule_partitions_every_tile(name, wgs):
    hidden, inter, ks, ff, af, on = LAYERS[name]
    L = _layer(hidden, inter, ks, ff, af, on)
    rows = _rows(hidden, inter)
    rec = spax.layer_schedule(L, wgs)
    assert rec.shape[1] == 9 and len(rec) > 0
    w, g, t, f0, f1, a0, a1, wlo, whi = rec.T
    assert w.min() >= 0 and w.max() < wgs
    present = [grp for grp in range(4) if on[grp]]
    assert set(np.unique(g)) == set(present)
    for grp in present:
        kf, ka = ks[grp]
        tiles = (rows[grp] + TILE - 1) // TILE
        sel = g == grp
        assert set(np.unique(t[sel])) == set(range(tiles)), "every tile is met"
        wg = np.unique(w[sel])
        if kf + ka > 0:
            # a contiguous range of workgroups; slot t + i distinct and in range
            assert list(wg) == list(range(wg[0], wg[-1] + 1))
            slots = t[sel] + (w[sel] - wg[0])
            assert len(np.unique(slots)) == sel.sum() and slots.max() < tiles + len(wg)
        else:
            # no selected columns: each tile once, dealt round-robin
            assert sel.sum() == tiles and np.all(wlo[sel] == w[sel]) and np.all(whi[sel] == w[sel])
        for tt in range(tiles):
            m = sel & (t == tt)
            order = np.argsort(w[m])
            ws_, F0, F1, A0, A1 = w[m][order], f0[m][order], f1[m][order], a0[m][order], a1[m][order]
            # the same contributors named by every contributor, and exactly them
            assert len(np.unique(wlo[m])) == 1 and len(np.unique(whi[m])) == 1
            assert list(ws_) == list(range(wlo[m][0], whi[m][0] + 1))
            # the tier lists are cut into consecutive pieces covering them exactly
            assert F0[0] == 0 and F1[-1] == kf and A0[0] == 0 and A1[-1] == ka
            assert np.all(F1[:-1] == F0[1:]) and np.all(A1[:-1] == A0[1:])
            assert np.all(F1 >= F0) and np.all(A1 >= A0)
    # each workgroup visits the groups in processing order, tiles ascending
    rank = {grp: i for i, grp in enumerate(ORDER)}
    for ww in range(wgs):
        m = w == ww
        key = [(rank[a], b) for a, b in zip(g[m], t[m])]
        assert key == sorted(key)
    # q/k/v and o never share a workgroup when both have columns and there
    # are two workgroups or more
    if on[spax.GROUP_QKV] and on[spax.GROUP_O] and sum(ks[0]) and sum(ks[1]) and wgs >= 2:
        assert not set(w[g == spax.GROUP_QKV]) & set(w[g == spax.GROUP_O])


@pytest.mark.parametrize("wgs", [37, 256])
@pytest.mark.parametrize("name", ["7b", "70b_ffn"])
def test_schedule_balances_bytes(name, wgs):
    hidden, inter, ks, ff, af, on = LAYERS[name]
    L = _layer(hidden, inter, ks, ff, af, on)
    rec = spax.layer_schedule(L, wgs)
    w, g, t, f0, f1, a0, a1 = rec.T[:7]
    cost = (f1 - f0) * _tile_bytes(ff) + (a1 - a0) * _tile_bytes(af)
    unit = max(_tile_bytes(ff), _tile_bytes(af))
    per_wg = {}
    for grp in range(4):
        sel = g == grp
        if not sel.any():
            continue
        wg = np.unique(w[sel])
        per = np.array([cost[sel & (w == ww)].sum() for ww in wg])
        nseg = max(int((sel & (w == ww)).sum()) for ww in wg)
        # runs differ by one unit; each segment rounds each tier by one column
        assert per.max() - per.min() <= (1 + 2 * nseg) * unit, (grp, per.min(), per.max())
        per_wg[grp] = per.mean()
        if grp in (spax.GROUP_GATE_UP, spax.GROUP_DOWN):
            assert len(wg) == wgs
    if spax.GROUP_QKV in per_wg and spax.GROUP_O in per_wg:
        # q/k/v and o end together: their ranges are in proportion to bytes
        nq = len(np.unique(w[g == spax.GROUP_QKV]))
        no = len(np.unique(w[g == spax.GROUP_O]))
        assert nq + no == wgs
        ratio = per_wg[spax.GROUP_QKV] / per_wg[spax.GROUP_O]
        assert abs(ratio - 1.0) <= 1.0 / min(nq, no) + 0.02, ratio


def test_schedule_rejects_what_the_layer_kernel_does_not_run():
    hidden, inter, ks, ff, af, on = LAYERS["7b"]
    L = _layer(hidden, inter, ks, spax.FMT_FP16, spax.FMT_INT4_G128, on)
    with pytest.raises(spax.SpaxError):
        spax.layer_schedule(L, 513)            # more workgroups than the partials hold
    L = _layer(hidden, inter, ks, spax.FMT_FP16, spax.FMT_INT4_G128, on)
    L.group[1] = _m(hidden, hidden, spax.FMT_FP16, spax.FMT_INT2_G128)
    with pytest.raises(spax.SpaxError):
        spax.layer_schedule(L, 256)            # two format pairs in one layer
    L = _layer(hidden, inter, ks, spax.FMT_INT4_G128, spax.FMT_INT2_G128, on)
    with pytest.raises(spax.SpaxError):
        spax.layer_schedule(L, 256)            # an int4 full tier: per-group launches
    big = _layer(4096, 11008, [(8192, 8192), (1024, 1024), (1024, 1024), (2752, 2752)])
    with pytest.raises(spax.SpaxError):
        spax.layer_schedule(big, 256)          # lists past the LDS capacity
