"""The trellis-coded middle tier on the GPU (SpAx page section 5.1) against
the oracle: the list-reading product (codebook in LDS), the layer step (which
ranks separately for this tier) and the host-resident mode.

The codes come from the library's offline host encoder, which is pinned bit
for bit against the oracle's encoder on the CPU (tests/test_oracle_trellis.py;
rechecked here on one small case); the oracle then rebuilds the columns from
those codes itself."""
import numpy as np
import pytest

import oracle as O
import oracle.spax_trellis as T
import workloads as WL
from tests.spax_testlib import (RowsOf, SegmentedStore, TrellisStore, check_product, log,
                                 sample_groups, split_codes, to_dev,
                                 to_host)

pytestmark = pytest.mark.gpu


def _matrix(Wt, residency=0):
    import activation_sparse_decode_token_amd as spax
    from activation_sparse_decode_token_amd.layouts import build_matrix
    cb = WL.trellis_codebook(1)
    W = build_matrix(to_dev(Wt), spax.FMT_FP16, spax.FMT_TRELLIS, residency=residency,
                     codebook=to_dev(cb))
    codes = to_host(W._keep[2]) if residency == 0 else W._keep[2].numpy()
    scales = to_host(W._keep[3]) if residency == 0 else W._keep[3].numpy()
    return W, TrellisStore(codes, scales, cb)


def _run(W, x16, F, A, ws=None, copy=None):
    import torch
    import activation_sparse_decode_token_amd as spax
    dev = torch.device("cuda:0")
    if ws is None:
        ws = torch.zeros(spax.gemv_workspace_bytes(W), dtype=torch.uint8, device=dev)
    y = torch.full((W.rows,), 0x7E00, dtype=torch.int16, device=dev)
    Fd = to_dev(F.astype(np.int32)) if len(F) else torch.zeros(1, dtype=torch.int32, device=dev)
    Ad = to_dev(A.astype(np.int32)) if len(A) else torch.zeros(1, dtype=torch.int32, device=dev)
    spax.tiered_gemv(W, to_dev(x16), Fd, len(F), Ad, len(A), y, ws, copy=copy)
    torch.cuda.synchronize()
    return to_host(y).view(np.float16), ws


def test_host_encoder_matches_oracle_encoder():
    Wt = WL.weights_fp16(850, 0, "w", 128, 3, 0.02)
    _, st = _matrix(Wt)
    oc, os_ = T.pack_trellis(Wt, WL.trellis_codebook(1))
    assert np.array_equal(st.codes, oc)
    assert np.array_equal(st.scales.view(np.uint16), os_.view(np.uint16))


CASES = [
    # R, n, k_full, k_approx
    (640, 300, 60, 90),       # ragged last tile (512 + 128)
    (1536, 200, 50, 80),
    (512, 7, 3, 4),
    (3072, 128, 0, 128),      # all approx
    (1024, 256, 64, 64),
]


@pytest.mark.parametrize("R,n,kf,ka", CASES)
def test_trellis_product_vs_oracle(R, n, kf, ka):
    log(f"trellis R={R} n={n} kf={kf} ka={ka}")
    Wt = WL.weights_fp16(851, R, "w", R, n, 0.02)
    Wt[0] = 0                               # a zero column: scale 0
    x = WL.laplace_fp16(851, R, "x", n, n)
    F, A = O.plan_tiers(x, kf, ka)
    W, st = _matrix(Wt)
    y, ws = _run(W, x, F, A)
    err = check_product(y, x, F, A, O.ColumnStore("fp16", Wt), st, f"trellis R={R} n={n}")
    y2, _ = _run(W, x, F, A, ws)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    log(f"  norm-wise error {err:.2e}")


@pytest.mark.parametrize("choice", [0, 1, 2])
def test_trellis_layer_step(choice):
    """A one-group layer with the trellis tier, under each launch form (the
    layer kernel does not take the trellis tier: AUTO runs the per-group
    launch)."""
    import torch
    import activation_sparse_decode_token_amd as spax
    if True:
        R, n = 1024, 512
        Wt = WL.weights_fp16(852, 0, "w", R, n, 0.02)
        W, st = _matrix(Wt)
        kf, ka = WL.tier_counts(n, WL.TierSplit(40, 30, 30))
        L = spax.Layer.make([W, None, None, None], [kf, 0, 0, 0], [ka, 0, 0, 0], kernel=choice)
        dev = torch.device("cuda:0")
        ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device=dev)
        for tok in range(2):
            x = WL.laplace_fp16(852, 0, "x", tok, n)
            Fd = torch.empty(kf, dtype=torch.int32, device=dev)
            Ad = torch.empty(ka, dtype=torch.int32, device=dev)
            y = torch.empty(R, dtype=torch.float16, device=dev)
            io = spax.LayerIO.make(h=to_dev(x), qkv=y, full_idx=(Fd, None, None, None),
                                   approx_idx=(Ad, None, None, None))
            spax.layer_step(L, io, ws)
            torch.cuda.synchronize()
            F, A = O.plan_tiers(x, kf, ka)
            assert np.array_equal(to_host(Fd), F) and np.array_equal(to_host(Ad), A)
            check_product(to_host(y), x, F, A, O.ColumnStore("fp16", Wt), st,
                          f"trellis layer token {tok}")


def test_trellis_host_pinned_bitwise_equals_device():
    import torch
    R, n = 1536, 384
    Wt = WL.weights_fp16(853, 0, "w", R, n, 0.02)
    Wd, st = _matrix(Wt)
    Wh, sth = _matrix(Wt, residency=1)
    assert np.array_equal(st.codes, sth.codes)
    import activation_sparse_decode_token_amd as spax
    cs = spax.copy_init(torch.cuda.Stream())
    for tok in range(2):
        x = WL.laplace_fp16(853, 0, "x", tok, n)
        F, A = O.plan_tiers(x, 100, 150)
        yd, _ = _run(Wd, x, F, A)
        yh, _ = _run(Wh, x, F, A, copy=cs)
        assert np.array_equal(yd.view(np.uint16), yh.view(np.uint16)), tok
    spax.copy_release(cs)
    log("trellis host-pinned == device bitwise")


@pytest.mark.parametrize("R,n,kf,ka", [(640, 300, 60, 90), (256, 2000, 500, 600),
                                       (1152, 513, 100, 300)])
def test_trellis_fused_ranking(R, n, kf, ka):
    """A one-group layer step with the trellis tier and device-resident
    weights: the product ranks x itself (list piece of at most 1024 positions
    beside the LDS codebook); lists bit-exact, product within the bound."""
    import torch
    import activation_sparse_decode_token_amd as spax
    Wt = WL.weights_fp16(854, R, "w", R, n, 0.02)
    W, st = _matrix(Wt)
    L = spax.Layer.make([W, None, None, None], [kf, 0, 0, 0], [ka, 0, 0, 0])
    dev = torch.device("cuda:0")
    ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device=dev)
    x = WL.laplace_fp16(854, R, "x", 0, n)
    Fd = torch.full((kf + 8,), -7, dtype=torch.int32, device=dev)
    Ad = torch.full((ka + 8,), -7, dtype=torch.int32, device=dev)
    y = torch.empty(R, dtype=torch.float16, device=dev)
    io = spax.LayerIO.make(h=to_dev(x), qkv=y, full_idx=(Fd, None, None, None),
                           approx_idx=(Ad, None, None, None))
    spax.layer_step(L, io, ws)
    torch.cuda.synchronize()
    F, A = O.plan_tiers(x, kf, ka)
    Fh, Ah = to_host(Fd), to_host(Ad)
    assert np.array_equal(Fh[:kf], F) and np.array_equal(Ah[:ka], A)
    assert np.all(Fh[kf:] == -7) and np.all(Ah[ka:] == -7)
    err = check_product(to_host(y), x, F, A, O.ColumnStore("fp16", Wt), st,
                        f"trellis fused R={R} n={n}")
    log(f"trellis fused R={R} n={n}: norm-wise error {err:.2e}")


def test_gpu_encoder_matches_oracle_and_host_encoder():
    """spax_pack_trellis (the Viterbi on the GPU) against the oracle on small
    columns with special cases, and against the host encoder (itself pinned
    to the oracle) on a larger matrix, in several launches."""
    import torch
    import activation_sparse_decode_token_amd as spax
    dev = torch.device("cuda:0")
    cb = WL.trellis_codebook(1)
    rs = np.random.default_rng(855)
    Wt = WL.weights_fp16(855, 0, "w", 256, 6, 0.02)
    Wt[0] = 0                                                        # zero column
    Wt[1, 9] = np.float16(5.0)                                       # an outlier
    Wt[2] = (rs.integers(-30, 31, 256) * 2.0 ** -24).astype(np.float16)  # subnormal
    Wt[3] = (rs.choice([-1.0, 1.0], 256) * 0.25).astype(np.float16)  # one magnitude

    def gpu(W, per_launch):
        n, R = W.shape
        codes = torch.empty((n, R // 4), dtype=torch.uint8, device=dev)
        scales = torch.empty(n, dtype=torch.float16, device=dev)
        ws = torch.empty(spax.pack_trellis_workspace_bytes(R, per_launch), dtype=torch.uint8,
                         device=dev)
        spax.pack_trellis(to_dev(W), R, n, to_dev(cb), codes, scales, ws)
        torch.cuda.synchronize()
        return to_host(codes), to_host(scales)

    c, s = gpu(Wt, 4)                      # two launches
    oc, os_ = T.pack_trellis(Wt, cb)
    assert np.array_equal(s.view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(c, oc)
    W2 = WL.weights_fp16(856, 0, "w", 1024, 48, 0.02)
    c2, s2 = gpu(W2, 20)                   # three launches
    hc = np.zeros((48, 256), dtype=np.uint8)
    hs = np.zeros(48, dtype=np.float16)
    spax.pack_trellis_host(W2, 1024, 48, cb, hc, hs)
    assert np.array_equal(s2.view(np.uint16), hs.view(np.uint16))
    assert np.array_equal(c2, hc)
    log("GPU trellis encoder == oracle / host encoder")


def test_full_size_7b_attention_trellis():
    """The 7B attention projections with the trellis tier at full size (o:
    4096 x 4096; q, k, v stacked: 12288 x 4096; 40/30/30 %), in the launch the
    benchmark times (a one-group layer step, which ranks x inside the
    product; codes from the GPU encoder): lists bit-exact; whole 128-row
    groups of y against the oracle, which rebuilds those columns from the
    codes itself (q, k and v each as its own matrix column)."""
    import torch
    import activation_sparse_decode_token_amd as spax
    import activation_sparse_decode_token_amd.layouts as LY
    from activation_sparse_decode_token_amd.layouts import build_matrix
    dev = torch.device("cuda:0")
    cb = WL.trellis_codebook(1)
    n = 4096
    kf, ka = WL.tier_counts(n, WL.CONFIGS[2].splits[0])
    saved = LY.TRELLIS_WS_BYTES
    LY.TRELLIS_WS_BYTES = 8 << 30    # backpointers of 160+ columns per encoder launch
    try:
        for R, stacked, label in [(4096, None, "7B o-proj trellis"),
                                  (12288, ("q", "k", "v"), "7B qkv stacked trellis")]:
            if stacked is None:
                Wt = WL.weights_fp16(2, 0, "w", R, n, 0.02)
            else:
                Wt = np.concatenate([WL.weights_fp16(2, 0, m, R // 3, n, 0.02) for m in stacked],
                                    axis=1)
            nm = 1 if stacked is None else 3
            W = build_matrix(to_dev(Wt), spax.FMT_FP16, spax.FMT_TRELLIS, codebook=to_dev(cb),
                             seg_rows=0 if stacked is None else R // 3)
            codes, scales = to_host(W._keep[2]), to_host(W._keep[3])
            if nm == 1:
                st = TrellisStore(codes, scales, cb)
            else:
                # q, k and v are coded as their own columns (SpAx page 5.1)
                st = SegmentedStore([TrellisStore(c, sc, cb)
                                     for c, sc in split_codes(codes, scales, nm)])
            rows = sample_groups(R, 8, 14 + R)
            full = O.ColumnStore("fp16", np.ascontiguousarray(Wt[:, rows]))
            L = spax.Layer.make([W, None, None, None], [kf, 0, 0, 0], [ka, 0, 0, 0])
            ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device=dev)
            Fd = torch.empty(kf, dtype=torch.int32, device=dev)
            Ad = torch.empty(ka, dtype=torch.int32, device=dev)
            y = torch.empty(R, dtype=torch.float16, device=dev)
            x = WL.laplace_fp16(2, 0, "x", 0, n)
            io = spax.LayerIO.make(h=to_dev(x), qkv=y, full_idx=(Fd, None, None, None),
                                   approx_idx=(Ad, None, None, None))
            spax.layer_step(L, io, ws)
            torch.cuda.synchronize()
            F, A = O.plan_tiers(x, kf, ka)
            assert np.array_equal(to_host(Fd), F) and np.array_equal(to_host(Ad), A), label
            err = check_product(to_host(y), x, F, A, full, RowsOf(st, rows), label, rows=rows)
            assert np.all(np.isfinite(to_host(y).astype(np.float32)))
            log(f"{label}: norm-wise error {err:.2e} (kf={kf} ka={ka})")
    finally:
        LY.TRELLIS_WS_BYTES = saved
