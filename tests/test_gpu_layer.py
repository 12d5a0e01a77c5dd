"""spax_layer_step and the host-resident mode on the GPU."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from tests.spax_testlib import (RowsOf, SegmentedStore, TrellisStore, check_product, log,
                                sample_groups, split_codes, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _spax():
    import activation_sparse_decode_token_amd as spax
    return spax


class LayerWeights:
    """Column-major fp16 weights of one layer, drawn on the host."""

    def __init__(self, cfg, layer, hidden, inter, std, attn=True):
        self.hidden, self.inter = hidden, inter
        self.q = self.k = self.v = self.o = None
        if attn:
            self.q = WL.weights_fp16(cfg, layer, "q", hidden, hidden, std)
            self.k = WL.weights_fp16(cfg, layer, "k", hidden, hidden, std)
            self.v = WL.weights_fp16(cfg, layer, "v", hidden, hidden, std)
            self.o = WL.weights_fp16(cfg, layer, "o", hidden, hidden, std)
        self.gate = WL.weights_fp16(cfg, layer, "gate", inter, hidden, std)
        self.up = WL.weights_fp16(cfg, layer, "up", inter, hidden, std)
        self.down = WL.weights_fp16(cfg, layer, "down", hidden, inter, std)


def _build_layer(w: LayerWeights, ff, af, residency, ks, kernel=0):
    import torch
    spax = _spax()
    from activation_sparse_decode_token_amd.layouts import build_matrix, glu_interleave, stack_rows
    F = {"fp16": 1, "int4": 2}[ff]
    A = {"int4": 2, "int2": 3, "sign2": 4, "trellis": 5}[af]
    cb = to_dev(WL.trellis_codebook(2)) if af == "trellis" else None
    qkv = o = None
    if w.q is not None:
        qkv = build_matrix(stack_rows([to_dev(w.q), to_dev(w.k), to_dev(w.v)]), F, A,
                           residency=residency, codebook=cb, seg_rows=w.hidden)
        o = build_matrix(to_dev(w.o), F, A, residency=residency, codebook=cb)
    gu = build_matrix(glu_interleave(to_dev(w.gate), to_dev(w.up)), F, A,
                      layout=spax.LAYOUT_GLU_INTERLEAVED, residency=residency, codebook=cb)
    dn = build_matrix(to_dev(w.down), F, A, residency=residency, codebook=cb)
    torch.cuda.synchronize()
    kf = [ks[g][0] for g in ("qkv", "o", "ffn", "down")]
    ka = [ks[g][1] for g in ("qkv", "o", "ffn", "down")]
    return spax.Layer.make([qkv, o, gu, dn], kf, ka, kernel=kernel)


def _io(L, h, z, x):
    import torch
    spax = _spax()
    dev = torch.device("cuda:0")
    G = L.group
    out = {
        "qkv": torch.empty(max(1, G[0].rows), dtype=torch.float16, device=dev),
        "o": torch.empty(max(1, G[1].rows), dtype=torch.float16, device=dev),
        "g": torch.empty(G[2].rows // 2, dtype=torch.float16, device=dev),
        "u": torch.empty(G[2].rows // 2, dtype=torch.float16, device=dev),
        "a": torch.empty(G[2].rows // 2, dtype=torch.float16, device=dev),
        "down": torch.empty(G[3].rows, dtype=torch.float16, device=dev),
        "F": [torch.empty(max(1, L.k_full[g]), dtype=torch.int32, device=dev) for g in range(4)],
        "A": [torch.empty(max(1, L.k_approx[g]), dtype=torch.int32, device=dev) for g in range(4)],
    }
    io = spax.LayerIO.make(h=None if h is None else to_dev(h), z=None if z is None else to_dev(z),
                           x=to_dev(x), qkv=out["qkv"], o=out["o"],
                           g=out["g"], u=out["u"], a=out["a"], down=out["down"],
                           full_idx=out["F"], approx_idx=out["A"])
    return io, out


def _run_layer(L, h, z, x, ws=None, copy=None):
    import torch
    spax = _spax()
    if ws is None:
        ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device="cuda:0")
    io, out = _io(L, h, z, x)
    spax.layer_step(L, io, ws, copy=copy)
    torch.cuda.synchronize()
    assert spax.workspace_status(ws) == 0, "a bounded wait of the layer kernel ran out"
    torch.cuda.synchronize()
    res = {k: to_host(out[k]) for k in ("qkv", "o", "g", "u", "a", "down")}
    res["lists"] = [(to_host(out["F"][g])[:L.k_full[g]], to_host(out["A"][g])[:L.k_approx[g]])
                    for g in range(4)]
    return res, ws


def _check_layer(res, w: LayerWeights, ks, h, z, x, ff, af, label, rows_per=None, L=None):
    """Stage-wise parity: each group is compared with the oracle fed the same
    inputs the GPU group saw (down is fed the GPU's a)."""
    def stores(Wt, rows=None, parts=None, lib=None):
        """Oracle stores of the matrix Wt (its rows `rows`). The sign and
        trellis codes are per matrix column (SpAx page section 5.1): for the
        stacked q/k/v, `parts` are q, k, v, each coded on its own; gate and
        up are checked as their own matrices. The trellis store rebuilds
        the library's codes of each matrix (its encoder is pinned to the
        oracle's), `lib` = [(codes, scales)] per matrix."""
        sub = Wt if rows is None else np.ascontiguousarray(Wt[:, rows])
        if af not in ("sign2", "trellis"):
            return O.ColumnStore(ff, sub), O.ColumnStore(af, sub)
        if af == "sign2":
            per = []
            for p in (parts or [Wt]):
                c, sc = O.pack_sign2(p)
                per.append(O.ColumnStore("sign2", codes=c, scales=sc))
        else:
            per = [TrellisStore(c, sc, cbh) for c, sc in lib]
        approx = SegmentedStore(per) if len(per) > 1 else per[0]
        if rows is not None:
            approx = RowsOf(approx, rows)
        return O.ColumnStore(ff, sub), approx

    attn = w.q is not None
    Wqkv = np.concatenate([w.q, w.k, w.v], axis=1) if attn else None
    lib = {}
    if af == "trellis":
        cbh = WL.trellis_codebook(2)
        for g, n_mat, lay in ((0, 3, "stacked"), (1, 1, "stacked"), (2, 2, "glu"),
                              (3, 1, "stacked")):
            if g < 2 and not attn:
                continue
            keep = L._keep[g]._keep
            codes, scales = to_host(keep[2]), to_host(keep[3])
            lib[g] = (split_codes(codes, scales, n_mat, lay) if n_mat > 1
                      else [(codes, scales if scales.ndim == 1 else scales[:, 0])])

    if attn:
        L0 = O.plan_tiers(h, *ks["qkv"])
        assert all(np.array_equal(a, b) for a, b in zip(res["lists"][0], L0)), \
            f"{label}: qkv lists"
        rows = sample_groups(Wqkv.shape[1], 8, 1) if rows_per else None
        check_product(res["qkv"], h, *L0,
                      *stores(Wqkv, rows, parts=[w.q, w.k, w.v], lib=lib.get(0)),
                      f"{label} qkv", rows=rows)

        L1 = O.plan_tiers(z, *ks["o"])
        assert all(np.array_equal(a, b) for a, b in zip(res["lists"][1], L1)), \
            f"{label}: o lists"
        rows = sample_groups(w.o.shape[1], 8, 2) if rows_per else None
        check_product(res["o"], z, *L1, *stores(w.o, rows, lib=lib.get(1)), f"{label} o",
                      rows=rows)

    L2 = O.plan_tiers(x, *ks["ffn"])
    assert all(np.array_equal(a, b) for a, b in zip(res["lists"][2], L2)), f"{label}: ffn lists"
    rows = sample_groups(w.inter, 8, 3) if rows_per else None
    check_product(res["g"], x, *L2, *stores(w.gate, rows, lib=lib[2][:1] if lib else None),
                  f"{label} gate", rows=rows)
    check_product(res["u"], x, *L2, *stores(w.up, rows, lib=lib[2][1:] if lib else None),
                  f"{label} up", rows=rows)
    # a is formed from the GPU's own fp16 g and u
    a_want = O.swiglu_fp16(res["g"], res["u"]).astype(np.float64)
    a_got = res["a"].astype(np.float64)
    scale = np.abs(a_want).max()
    assert np.abs(a_got - a_want).max() <= 2e-3 * scale, f"{label}: a"
    assert np.all(np.abs(a_got - a_want) <= 2.0 ** -10 * np.abs(a_want) + 2.0 ** -24), \
        f"{label}: a off by more than one fp16 ulp"

    L3 = O.plan_tiers(res["a"], *ks["down"])
    assert all(np.array_equal(a, b) for a, b in zip(res["lists"][3], L3)), f"{label}: down lists"
    rows = sample_groups(w.hidden, 8, 4) if rows_per else None
    check_product(res["down"], res["a"], *L3, *stores(w.down, rows, lib=lib.get(3)),
                  f"{label} down", rows=rows)


def _ks(hidden, inter, split):
    return {"qkv": WL.tier_counts(hidden, split), "o": WL.tier_counts(hidden, split),
            "ffn": WL.tier_counts(hidden, split), "down": WL.tier_counts(inter, split)}


@pytest.mark.parametrize("ff,af", [("fp16", "int4"), ("int4", "int2"), ("fp16", "int2"),
                                   ("fp16", "sign2"), ("fp16", "trellis")])
def test_layer_small(ff, af, kernel_choice):
    hidden, inter = 512, 1408          # ragged tiles: 1408 = 2*512 + 384; gate/up 2816 rows
    w = LayerWeights(810, 0, hidden, inter, 0.02)
    ks = _ks(hidden, inter, WL.TierSplit(40, 30, 30))
    L = _build_layer(w, ff, af, 0, ks, kernel_choice)
    for tok in range(3):
        h = WL.laplace_fp16(810, 0, "h", tok, hidden)
        z = WL.laplace_fp16(810, 0, "z", tok, hidden)
        x = WL.laplace_fp16(810, 0, "x", tok, hidden)
        res, _ = _run_layer(L, h, z, x)
        _check_layer(res, w, ks, h, z, x, ff, af, f"small {ff}/{af} token {tok}", L=L)
    log(f"layer small {ff}/{af} ok")


@pytest.mark.parametrize("wgs", [1, 2, 5, 37])
def test_layer_kernel_workgroup_caps(wgs):
    """The layer kernel on a few workgroups: each one meets many row tiles of
    a group (several segments per group, the ranking then places whole
    lists), and at one workgroup q/k/v and o share it."""
    hidden, inter = 512, 1408
    w = LayerWeights(811, 0, hidden, inter, 0.02)
    ks = _ks(hidden, inter, WL.TierSplit(40, 30, 30))
    L = _build_layer(w, "fp16", "int4", 0, ks, 0)
    L.workgroups = wgs
    for tok in range(2):
        h = WL.laplace_fp16(811, 0, "h", tok, hidden)
        z = WL.laplace_fp16(811, 0, "z", tok, hidden)
        x = WL.laplace_fp16(811, 0, "x", tok, hidden)
        res, _ = _run_layer(L, h, z, x)
        _check_layer(res, w, ks, h, z, x, "fp16", "int4", f"{wgs} workgroups token {tok}")
    log(f"layer kernel on {wgs} workgroups ok")


def test_layer_kernel_7b_on_37_workgroups():
    """A full-size 7B layer on 37 workgroups: runs of units that cross many
    tiles, contributors that differ per tile."""
    w = LayerWeights(4, 0, 4096, 11008, 0.02)
    ks = _ks(4096, 11008, WL.CONFIGS[4].splits[0])
    L = _build_layer(w, "fp16", "int4", 0, ks, 0)
    L.workgroups = 37
    h = WL.laplace_fp16(4, 0, "h", 0, 4096)
    z = WL.laplace_fp16(4, 0, "z", 0, 4096)
    x = WL.laplace_fp16(4, 0, "x", 0, 4096)
    res, _ = _run_layer(L, h, z, x)
    _check_layer(res, w, ks, h, z, x, "fp16", "int4", "7B layer on 37 workgroups", rows_per=True)
    log("7B layer on 37 workgroups ok")


def _tied(case, seed, n):
    """Inputs with many equal magnitudes: the ranking's ties (lower index
    first) decide most of the lists."""
    rs = np.random.default_rng(seed)
    if case == "all-equal":
        return np.full(n, -1.5, dtype=np.float16)
    if case == "signed-zeros":
        return rs.choice(np.array([0.0, -0.0], dtype=np.float16), n)
    if case == "small-alphabet":
        return rs.choice(np.array([0, -0.0, 1, -1, 2, -2, 0.5], dtype=np.float16), n)
    if case == "subnormal":
        return (rs.integers(-3, 4, n) * 2.0 ** -24).astype(np.float16)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["all-equal", "signed-zeros", "small-alphabet", "subnormal"])
def test_layer_kernel_tied_inputs(case):
    """The layer kernel's rankings on inputs full of ties, with empty tiers,
    tiers that take every column, and a ragged last round of 512 entries
    (down's input has 1408 entries): lists equal the oracle's exactly."""
    hidden, inter = 512, 1408
    w = LayerWeights(812, 0, hidden, inter, 0.02)
    for ks in ({"qkv": (128, 128), "o": (0, 200), "ffn": (256, 0), "down": (1, 1406)},
               {"qkv": (511, 1), "o": (170, 171), "ffn": (0, 512), "down": (704, 0)}):
        L = _build_layer(w, "fp16", "int4", 0, ks, 0)
        assert len(_spax().layer_schedule(L, 256)) > 0  # the one-launch layer kernel runs
        h, z, x = (_tied(case, 812 + i, hidden) for i in range(3))
        res, _ = _run_layer(L, h, z, x)
        _check_layer(res, w, ks, h, z, x, "fp16", "int4", f"tied {case} {ks}")
    log(f"layer kernel on tied inputs ({case}) ok")


def test_layer_kernel_ragged_down_many_contributors():
    """Down with a ragged last row tile (640 rows: 512 + 128) whose tiles
    have far more than 32 contributors (every workgroup meets both): the
    last eight contributors to arrive share each tile's final sum in 64-row
    slices, slices past the last row store nothing, and the partials are
    loaded in batches of 32 contributors."""
    hidden, inter = 640, 5632          # an FFN layer (stacked q/k/v take whole tiles)
    w = LayerWeights(813, 0, hidden, inter, 0.02, attn=False)
    ks = _ks(hidden, inter, WL.TierSplit(40, 30, 30))
    ks["qkv"] = ks["o"] = (0, 0)
    L = _build_layer(w, "fp16", "int4", 0, ks, 0)
    sched = _spax().layer_schedule(L, 256)
    assert len(sched) > 0  # the one-launch layer kernel runs
    down = sched[sched[:, 1] == _spax().GROUP_DOWN]
    assert sorted(set(down[:, 2])) == [0, 1]
    assert (down[:, 8] - down[:, 7] + 1).min() > 32, "tiles with more than 32 contributors"
    for tok in range(2):
        x = WL.laplace_fp16(813, 0, "x", tok, hidden)
        res, _ = _run_layer(L, None, None, x)
        _check_layer(res, w, ks, None, None, x, "fp16", "int4", f"ragged down token {tok}")
    log("layer kernel ragged down with many contributors ok")


@pytest.mark.parametrize("af", ["int4", "sign2"])
def test_layer_7b_shapes(kernel_choice, af):
    """A full-size 7B layer step (the launches the benchmarks time), with the
    int4 or the two-scale sign middle tier, on sampled whole row groups."""
    w = LayerWeights(4, 0, 4096, 11008, 0.02)
    ks = _ks(4096, 11008, WL.CONFIGS[4].splits[0])
    L = _build_layer(w, "fp16", af, 0, ks, kernel_choice)
    # (the oracle fits the sign code's scales over whole stored columns: one
    # token keeps that case short)
    for tok in ((0, 1) if af == "int4" else (0,)):
        h = WL.laplace_fp16(4, 0, "h", tok, 4096)
        z = WL.laplace_fp16(4, 0, "z", tok, 4096)
        x = WL.laplace_fp16(4, 0, "x", tok, 4096)
        res, _ = _run_layer(L, h, z, x)
        _check_layer(res, w, ks, h, z, x, "fp16", af, f"7B layer {af} token {tok}",
                     rows_per=True)
        log(f"7B layer {af} token {tok} ok")


@pytest.mark.parametrize("af", ["sign2", "trellis"])
def test_per_matrix_codes_of_stacked_and_glu_columns(af):
    """The sign and trellis codes of stacked q/k/v and GLU-interleaved
    gate/up stored columns are each matrix's own code: equal, matrix by
    matrix, to the oracle's packer (sign code) or encoder (trellis) applied
    to the unstacked matrix (SpAx page section 5.1: codes and scales per
    weight column, codes before the column start zero; section 5.3: stacked
    columns stay distinct columns)."""
    import oracle.spax_trellis as T
    spax = _spax()
    from activation_sparse_decode_token_amd.layouts import build_matrix, glu_interleave, stack_rows
    hidden, n = 512, 6 if af == "trellis" else 64
    A = {"sign2": spax.FMT_SIGN2, "trellis": spax.FMT_TRELLIS}[af]
    cb = WL.trellis_codebook(2)
    cbd = to_dev(cb) if af == "trellis" else None
    w = {m: WL.weights_fp16(812, 0, m, hidden, n, 0.02) for m in ("q", "k", "v", "gate", "up")}
    qkv = build_matrix(stack_rows([to_dev(w["q"]), to_dev(w["k"]), to_dev(w["v"])]),
                       spax.FMT_FP16, A, codebook=cbd, seg_rows=hidden)
    gu = build_matrix(glu_interleave(to_dev(w["gate"]), to_dev(w["up"])), spax.FMT_FP16, A,
                      layout=spax.LAYOUT_GLU_INTERLEAVED, codebook=cbd)
    assert qkv.approx_seg_rows == hidden
    for M, names, lay in ((qkv, ("q", "k", "v"), "stacked"), (gu, ("gate", "up"), "glu")):
        codes, scales = to_host(M._keep[2]), to_host(M._keep[3])
        assert scales.shape == (n, len(names) * (2 if af == "sign2" else 1))
        for (c, sc), m in zip(split_codes(codes, scales, len(names), lay), names):
            oc, os_ = O.pack_sign2(w[m]) if af == "sign2" else T.pack_trellis(w[m], cb)
            assert np.array_equal(c, oc), f"{af} codes of {m}"
            assert np.array_equal(np.asarray(sc).view(np.uint16),
                                  np.asarray(os_, dtype=np.float16).view(np.uint16)), \
                f"{af} scales of {m}"
    log(f"{af}: per-matrix codes of stacked q/k/v and GLU gate/up equal the oracle's")


def test_layer_70b_ffn_shapes(kernel_choice):
    """The config-5 launches at full size: the 57344-row GLU-interleaved
    int4/int2 gate/up with fused ranking and the SwiGLU epilogue, then the
    8192 x 28672 down ranked on the a it wrote (SpAx page sections 2 and
    5.2), on sampled whole row groups."""
    w = LayerWeights(5, 0, 8192, 28672, 0.015, attn=False)
    ks = _ks(8192, 28672, WL.CONFIGS[5].splits[0])
    L = _build_layer(w, "int4", "int2", 0, ks, kernel_choice)
    x = WL.laplace_fp16(5, 0, "x", 0, 8192)
    res, _ = _run_layer(L, None, None, x)
    _check_layer(res, w, ks, None, None, x, "int4", "int2", "70B FFN", rows_per=True)
    log(f"70B FFN layer step ok (kernel {kernel_choice})")


@pytest.mark.parametrize("ff,af", [("fp16", "int4"), ("int4", "int2"), ("fp16", "sign2")])
def test_host_pinned_bitwise_equals_device(ff, af):
    import torch
    hidden, inter = 1024, 2816
    w = LayerWeights(811, 0, hidden, inter, 0.02)
    ks = _ks(hidden, inter, WL.TierSplit(50, 25, 25))
    # host-resident groups run the per-group launches, which the device-resident
    # layer gives bit for bit under SPAX_KERNEL_PER_GROUP
    Ld = _build_layer(w, ff, af, 0, ks, kernel=2)
    Lh = _build_layer(w, ff, af, 1, ks)
    _host_vs_device(w, ks, Ld, Lh, ff, af, hidden)


def test_host_pinned_long_input():
    """Host-resident weights with an input past the one-workgroup ranking
    (down's 33024 inputs): the host branch that writes the sliced
    selection's lists for the copy, bitwise equal to the device-resident
    per-group launches and checked against the oracle."""
    hidden, inter = 512, 33024
    w = LayerWeights(811, 0, hidden, inter, 0.02, attn=False)
    ks = _ks(hidden, inter, WL.TierSplit(50, 25, 25))
    Ld = _build_layer(w, "fp16", "int4", 0, ks, kernel=2)
    Lh = _build_layer(w, "fp16", "int4", 1, ks)
    _host_vs_device(w, ks, Ld, Lh, "fp16", "int4", hidden)


def _host_vs_device(w, ks, Ld, Lh, ff, af, hidden):
    import torch
    spax = _spax()
    cs = spax.copy_init(torch.cuda.Stream())
    ws_d = ws_h = None
    for tok in range(3):
        h = WL.laplace_fp16(811, 0, "h", tok, hidden)
        z = WL.laplace_fp16(811, 0, "z", tok, hidden)
        x = WL.laplace_fp16(811, 0, "x", tok, hidden)
        rd, ws_d = _run_layer(Ld, h, z, x, ws_d)
        rh, ws_h = _run_layer(Lh, h, z, x, ws_h, copy=cs)
        for k in ("qkv", "o", "g", "u", "a", "down"):
            assert np.array_equal(rd[k].view(np.uint16), rh[k].view(np.uint16)), (k, tok)
        for g in range(4):
            for i in range(2):
                assert np.array_equal(rd["lists"][g][i], rh["lists"][g][i])
        if tok == 0:
            _check_layer(rh, w, ks, h, z, x, ff, af, f"host {ff}/{af}")
    spax.copy_release(cs)
    log(f"host-pinned {ff}/{af} == device bitwise")
