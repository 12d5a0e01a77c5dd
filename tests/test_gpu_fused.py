"""Fused tier selection + tiered product (spax_layer_step, device-resident
weights) against the oracle: bit-exact tier lists, products within tolerance.

A one-group layer (the QKV slot holding any matrix) runs exactly one fused
launch, so these cases cover the in-workgroup ranking on its own: ragged
input lengths, empty and full tiers, heavy ties, every format pair, ragged
row tiles, single-split and many-split launches, and the fallback to the
separate selection kernel past the fused kernel's input-length limit."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from tests.spax_testlib import check_product, log, to_dev, to_host

pytestmark = pytest.mark.gpu

FMT = {"fp16": 1, "int4": 2, "int2": 3, "sign2": 4, "none": 0}


def _one_group(Wt, x, ff, af, kf, ka, ws=None, kernel=0):
    import torch
    import activation_sparse_decode_token_amd as spax
    from activation_sparse_decode_token_amd.layouts import build_matrix
    dev = torch.device("cuda:0")
    n, R = Wt.shape
    W = build_matrix(to_dev(Wt), FMT[ff], FMT[af])
    L = spax.Layer.make([W, None, None, None], [kf, 0, 0, 0], [ka, 0, 0, 0], kernel=kernel)
    F = torch.full((max(kf, 1) + 8,), -7, dtype=torch.int32, device=dev)
    A = torch.full((max(ka, 1) + 8,), -7, dtype=torch.int32, device=dev)
    y = torch.full((R,), 0x7E00, dtype=torch.int16, device=dev)
    io = spax.LayerIO.make(h=to_dev(x), qkv=y, full_idx=(F, None, None, None),
                           approx_idx=(A, None, None, None))
    if ws is None:
        ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device=dev)
    spax.layer_step(L, io, ws)
    torch.cuda.synchronize()
    Fh, Ah = to_host(F), to_host(A)
    assert np.all(Fh[kf:] == -7) and np.all(Ah[ka:] == -7), "wrote past the lists"
    return to_host(y).view(np.float16), Fh[:kf], Ah[:ka], ws


def _check(Wt, x, ff, af, kf, ka, label, kernel=0):
    y, F, A, ws = _one_group(Wt, x, ff, af, kf, ka, kernel=kernel)
    oF, oA = O.plan_tiers(x, kf, ka)
    assert np.array_equal(F, oF), f"{label}: full list"
    assert np.array_equal(A, oA), f"{label}: approx list"
    full = O.ColumnStore(ff, Wt)
    approx = O.ColumnStore(af, Wt) if af != "none" else None
    err = check_product(y, x, oF, oA, full, approx, label)
    y2, F2, A2, _ = _one_group(Wt, x, ff, af, kf, ka, ws, kernel=kernel)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), f"{label}: not reproducible"
    return err


CASES = [
    # R, n, full, approx, kf, ka
    (128, 1, "fp16", "int4", 1, 0),
    (128, 2, "fp16", "int4", 0, 1),
    (256, 7, "fp16", "int4", 2, 3),
    (640, 300, "fp16", "int4", 60, 90),          # ragged tile, ragged x
    (1024, 1024, "fp16", "int4", 256, 256),      # single 1024x1024 layer, 50/25/25
    (1536, 1000, "fp16", "int2", 300, 300),
    (1152, 777, "int4", "int2", 100, 400),
    (1152, 777, "int4", "int4", 100, 400),
    (1024, 513, "int4", "none", 200, 0),
    (2048, 4096, "fp16", "none", 1229, 0),
    (3072, 2000, "fp16", "int4", 2000, 0),       # all full
    (3072, 2000, "fp16", "int4", 0, 2000),       # all approx
    (3072, 2000, "fp16", "int2", 0, 0),          # all skipped -> zeros
    (512, 4097, "fp16", "int4", 1000, 1500),     # one past a rank-width step
    (4096, 8192, "int4", "int2", 1638, 2458),
    (1024, 11008, "fp16", "int4", 2752, 2752),
    (640, 16385, "fp16", "int2", 4000, 6000),
    (1024, 28672, "int4", "int2", 5734, 8602),
    (512, 32768, "fp16", "int4", 9000, 9000),    # longest input ranked in one workgroup
    (512, 32769, "fp16", "int4", 9000, 9000),    # sliced selection, ragged last slice
    (256, 65536, "fp16", "int2", 20000, 30000),  # longest input: 16 slices
    (128, 6000, "fp16", "none", 6000, 0),        # one tile, one split, long list
    (640, 300, "fp16", "sign2", 60, 90),         # two-scale sign code
    (1024, 11008, "fp16", "sign2", 2752, 2752),
    (512, 32769, "fp16", "sign2", 9000, 9000),   # sliced selection
]


@pytest.mark.parametrize("R,n,ff,af,kf,ka", CASES)
def test_fused_vs_oracle(R, n, ff, af, kf, ka, kernel_choice):
    log(f"fused ({kernel_choice}) R={R} n={n} {ff}/{af} kf={kf} ka={ka}")
    Wt = WL.weights_fp16(820, R, "w", R, n, 0.02)
    x = WL.laplace_fp16(820, R, "x", n % 1000, n)
    err = _check(Wt, x, ff, af, kf, ka, f"R={R} n={n} {ff}/{af} kf={kf} ka={ka}",
                 kernel=kernel_choice)
    log(f"  norm-wise error {err:.2e}")


# 32768: the longest input one workgroup (or the layer kernel) ranks; 32769
# and 65536: past it, so the sliced selection and its placement (the layer
# kernel falls back to the per-group launches there)
@pytest.mark.parametrize("n", [300, 4096, 11008, 20000, 32768, 32769, 65536])
def test_fused_ties(n, kernel_choice):
    rs = np.random.default_rng(31 + n)
    Wt = WL.weights_fp16(821, 0, "w", 512, n, 0.02)
    cases = {
        "all-equal": np.full(n, -1.5, dtype=np.float16),
        "signed-zeros": rs.choice(np.array([0.0, -0.0], dtype=np.float16), n),
        "small-alphabet": rs.choice(np.array([0, -0.0, 1, -1, 2, -2, 0.5], dtype=np.float16), n),
        "subnormal": (rs.integers(-3, 4, n) * 2.0 ** -24).astype(np.float16),
    }
    for name, x in cases.items():
        for kf, ka in [(n // 4, n // 4), (n // 2, 0), (1, n - 1), (n // 3, n // 2)]:
            log(f"fused ties {name} n={n} kf={kf} ka={ka}")
            _check(Wt, x, "fp16", "int4", kf, ka, f"{name} n={n} kf={kf} ka={ka}",
                   kernel=kernel_choice)

