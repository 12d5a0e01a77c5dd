"""Packer and tiered gather-GEMV on the GPU vs the oracle."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from tests.spax_testlib import (check_product, log, sample_groups, to_dev, to_host)

pytestmark = pytest.mark.gpu

FMT = {"fp16": 1, "int4": 2, "int2": 3, "sign2": 4, "none": 0}


def _spax():
    import activation_sparse_decode_token_amd as spax
    return spax


def _device_matrix(Wt16, ff, af, layout=0):
    from activation_sparse_decode_token_amd.layouts import build_matrix
    return build_matrix(to_dev(Wt16), FMT[ff], FMT[af], layout=layout)


def _run(W, x16, F, A, ws=None):
    import torch
    spax = _spax()
    dev = torch.device("cuda:0")
    if ws is None:
        ws = torch.zeros(spax.gemv_workspace_bytes(W), dtype=torch.uint8, device=dev)
    y = torch.full((W.rows,), 0x7E00, dtype=torch.int16, device=dev)  # NaN pattern
    Fd = to_dev(F.astype(np.int32)) if len(F) else torch.zeros(1, dtype=torch.int32, device=dev)
    Ad = to_dev(A.astype(np.int32)) if len(A) else torch.zeros(1, dtype=torch.int32, device=dev)
    spax.tiered_gemv(W, to_dev(x16), Fd, len(F), Ad, len(A), y, ws)
    torch.cuda.synchronize()
    return to_host(y).view(np.float16), ws


@pytest.mark.parametrize("fmt", ["int4", "int2"])
@pytest.mark.parametrize("R,n", [(128, 3), (640, 77), (4096, 300)])
def test_pack_bit_exact(fmt, R, n):
    import torch
    from activation_sparse_decode_token_amd.layouts import pack
    Wt = WL.weights_fp16(801, 0, "w", R, n, 0.02)
    Wt[0] = 0                                   # an all-zero column
    Wt[1, :128] = np.float16(2.0 ** -20)        # a tiny group
    Wt[2, 5] = np.float16(7.0)                  # an outlier
    codes, scales = pack(to_dev(Wt), FMT[fmt])
    torch.cuda.synchronize()
    oc, os_ = (O.pack_int4_g128 if fmt == "int4" else O.pack_int2_g128)(Wt)
    assert np.array_equal(to_host(codes), oc)
    assert np.array_equal(to_host(scales).view(np.uint16), os_.view(np.uint16))


@pytest.mark.parametrize("R,n", [(128, 3), (640, 77), (4096, 300)])
def test_pack_sign2_bit_exact(R, n):
    """The two-scale sign packer against the oracle's: codes and both scales."""
    import torch
    from activation_sparse_decode_token_amd.layouts import pack
    rs = np.random.default_rng(R + n)
    Wt = WL.weights_fp16(804, 0, "w", R, n, 0.02)
    Wt[0] = 0                                                        # zero column
    Wt[1] = (rs.choice([-1.0, 1.0], R) * 0.375).astype(np.float16)   # one magnitude
    Wt[2] = (rs.integers(-8, 9, R) * 0.125).astype(np.float16)       # coarse grid: ties
    Wt[3 % n] = (rs.integers(-20, 21, R) * 2.0 ** -24).astype(np.float16)  # subnormal
    if n > 4:
        Wt[4, 5] = np.float16(7.0)                                   # an outlier
    codes, scales = pack(to_dev(Wt), FMT["sign2"])
    torch.cuda.synchronize()
    oc, os_ = O.pack_sign2(Wt)
    assert np.array_equal(to_host(scales).view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(to_host(codes), oc)


CASES = [
    # R, n, full fmt, approx fmt, k_full, k_approx
    (128, 64, "fp16", "int4", 10, 20),
    (640, 300, "fp16", "int4", 60, 90),       # ragged last tile (512 + 128)
    (1536, 1000, "fp16", "int2", 300, 300),
    (1152, 777, "int4", "int2", 100, 400),
    (1152, 777, "int4", "int4", 100, 400),
    (1024, 513, "int4", "none", 200, 0),
    (2048, 4096, "fp16", "none", 1229, 0),    # two tiers only (skip / full)
    (1024, 1024, "fp16", "int4", 256, 256),   # single 1024x1024 layer, 50/25/25
    (3072, 2000, "fp16", "int4", 2000, 0),    # all full == dense GEMV
    (3072, 2000, "fp16", "int4", 0, 2000),    # all approx
    (3072, 2000, "fp16", "int2", 0, 0),       # all skipped -> zeros
    (512, 7, "fp16", "int4", 3, 4),
    # more than 16 columns per wave on a ragged last tile (one split / capped splits)
    (1152, 777, "int4", "none", 100, 0),
    (1152, 777, "fp16", "int2", 0, 400),
    (640, 6000, "fp16", "none", 6000, 0),
    # the two-scale sign code as the approx tier
    (640, 300, "fp16", "sign2", 60, 90),
    (1536, 1000, "fp16", "sign2", 300, 300),
    (3072, 2000, "fp16", "sign2", 0, 2000),   # all approx
    (512, 7, "fp16", "sign2", 3, 4),
]


@pytest.mark.parametrize("R,n,ff,af,kf,ka", CASES)
def test_gemv_vs_oracle(R, n, ff, af, kf, ka):
    log(f"gemv R={R} n={n} {ff}/{af} kf={kf} ka={ka}")
    Wt = WL.weights_fp16(802, R, "w", R, n, 0.02)
    x = WL.laplace_fp16(802, R, "x", n, n)
    F, A = O.plan_tiers(x, kf, ka)
    W = _device_matrix(Wt, ff, af)
    y, ws = _run(W, x, F, A)
    full = O.ColumnStore(ff, Wt)
    approx = O.ColumnStore(af, Wt) if af != "none" else None
    err = check_product(y, x, F, A, full, approx, f"R={R} n={n} {ff}/{af}")
    # deterministic and leaves its workspace reusable: a second call is bitwise equal
    y2, _ = _run(W, x, F, A, ws)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    log(f"  norm-wise error {err:.2e}")


def test_gemv_unsorted_lists_and_fig2(golden_dir):
    import json
    import os
    g = json.load(open(os.path.join(golden_dir, "fig2_three_tier.json")))
    Wt = np.zeros((g["n"], g["rows"]), dtype=np.float16)
    Wt[:, :4] = np.array(g["columns_first4"], dtype=np.float16)
    x = np.array(g["x"], dtype=np.float16)
    W = _device_matrix(Wt, "fp16", "int4")
    y, _ = _run(W, x, np.array(g["expected_full"]), np.array(g["expected_approx"]))
    assert list(y[:4].astype(np.float64)) == g["expected_y_first4"]
    assert not np.any(y[4:].astype(np.float64))
    # list order does not change the selected set; the result stays within tolerance
    Wt2 = WL.weights_fp16(803, 0, "w", 1024, 900, 0.02)
    x2 = WL.laplace_fp16(803, 0, "x", 0, 900)
    F, A = O.plan_tiers(x2, 200, 300)
    rs = np.random.default_rng(1)
    W2 = _device_matrix(Wt2, "fp16", "int4")
    y2, _ = _run(W2, x2, rs.permutation(F), rs.permutation(A))
    check_product(y2, x2, F, A, O.ColumnStore("fp16", Wt2), O.ColumnStore("int4", Wt2), "perm")


def _full_size_case(cfg, R, n, ff, af, split, std, tokens, label, stacked=None):
    """Full-size projection; the oracle checks whole 128-row groups."""
    import torch
    spax = _spax()
    kf, ka = WL.tier_counts(n, split)
    if stacked is None:
        Wt = WL.weights_fp16(cfg, 0, "w", R, n, std)
    else:
        Wt = np.concatenate([WL.weights_fp16(cfg, 0, m, R // len(stacked), n, std)
                             for m in stacked], axis=1)
    W = _device_matrix(Wt, ff, af)
    ws = torch.zeros(spax.gemv_workspace_bytes(W), dtype=torch.uint8, device="cuda:0")
    rows = sample_groups(R, 12, cfg * 7 + R)
    sub = np.ascontiguousarray(Wt[:, rows])
    full = O.ColumnStore(ff, sub)
    if af == "sign2":
        # the sign code's scales are fitted over whole columns: pack all rows,
        # keep the codes of the sampled ones
        codes, scales = O.pack_sign2(Wt)
        approx = O.ColumnStore("sign2", codes=np.ascontiguousarray(codes[:, rows[0::4] // 4]),
                               scales=scales)
    else:
        approx = O.ColumnStore(af, sub) if af != "none" else None
    for tok in range(tokens):
        x = WL.laplace_fp16(cfg, 0, "x", tok, n)
        F, A = O.plan_tiers(x, kf, ka)
        y, _ = _run(W, x, F, A, ws)
        err = check_product(y, x, F, A, full, approx, f"{label} token {tok}", rows=rows)
        assert np.all(np.isfinite(y.astype(np.float32)))
        log(f"{label} token {tok}: norm-wise error {err:.2e} (kf={kf} ka={ka})")


def test_full_size_7b_attention():
    c = WL.CONFIGS[2]
    _full_size_case(2, 4096, 4096, "fp16", "int4", c.splits[0], 0.02, 2, "7B o-proj")
    _full_size_case(2, 12288, 4096, "fp16", "int4", c.splits[0], 0.02, 2, "7B qkv stacked",
                    stacked=("q", "k", "v"))


def test_full_size_7b_attention_sign2():
    c = WL.CONFIGS[2]
    _full_size_case(2, 4096, 4096, "fp16", "sign2", c.splits[0], 0.02, 1, "7B o-proj sign2")
    _full_size_case(2, 12288, 4096, "fp16", "sign2", c.splits[0], 0.02, 1,
                    "7B qkv stacked sign2", stacked=("q", "k", "v"))


@pytest.mark.parametrize("si", [0, 1, 2])
def test_full_size_7b_ffn(si):
    c = WL.CONFIGS[3]
    _full_size_case(3, 11008, 4096, "fp16", "int4", c.splits[si], 0.02, 1, f"7B gate s{si}")
    _full_size_case(3, 4096, 11008, "fp16", "int4", c.splits[si], 0.02, 1, f"7B down s{si}")


def test_full_size_70b_ffn():
    c = WL.CONFIGS[5]
    _full_size_case(5, 28672, 8192, "int4", "int2", c.splits[0], 0.015, 1, "70B gate")
    _full_size_case(5, 8192, 28672, "int4", "int2", c.splits[0], 0.015, 1, "70B down")


def test_workspace_shared_by_heights():
    """One workspace serves a tall matrix (80 row tiles, many splits) and a
    short one in turn: their partial sums and arrival counters must never
    overlap, whatever the heights."""
    import torch
    spax = _spax()
    tall = WL.weights_fp16(830, 0, "w", 40960, 256, 0.02)
    short = WL.weights_fp16(830, 1, "w", 512, 2048, 0.02)
    Wt = _device_matrix(tall, "fp16", "int4")
    Ws = _device_matrix(short, "fp16", "int4")
    ws = torch.zeros(max(spax.gemv_workspace_bytes(Wt), spax.gemv_workspace_bytes(Ws)),
                     dtype=torch.uint8, device="cuda:0")
    for rep in range(3):
        for Wd, Wh, n, label in ((Wt, tall, 256, "tall"), (Ws, short, 2048, "short")):
            x = WL.laplace_fp16(830, rep, "x", n, n)
            F, A = O.plan_tiers(x, n // 4, n // 4)
            y, ws = _run(Wd, x, F, A, ws)
            check_product(y, x, F, A, O.ColumnStore("fp16", Wh), O.ColumnStore("int4", Wh),
                          f"{label} rep {rep}")
    log("shared workspace ok")
