"""Pins for the trellis-code oracle (SpAx page section 5.1; no GPU): Viterbi
optimality by brute force, the window index by its closed form, exact
reconstruction where a zero-error path exists, the scale's closed forms."""
import itertools

import numpy as np

import oracle.spax_trellis as T
import workloads as WL


def _codebook(seed=5):
    return np.random.default_rng(seed).standard_normal(65536).astype(np.float16)


def test_window_index_closed_form():
    rs = np.random.default_rng(1)
    c = rs.integers(0, 4, 40)
    idx = T.trellis_indices(c)
    for i in range(40):
        want = sum(int(c[i - 7 + t]) * 4 ** t for t in range(8) if i - 7 + t >= 0)
        assert idx[i] == want
    # row 7 uses the codes of rows 0..7, row 8 those of rows 1..8
    assert idx[7] == sum(int(c[t]) * 4 ** t for t in range(8))
    assert idx[8] == sum(int(c[1 + t]) * 4 ** t for t in range(8))


def test_viterbi_is_optimal_by_brute_force():
    cb = _codebook(7)
    rs = np.random.default_rng(2)
    for trial in range(3):
        R = 8
        v = rs.standard_normal(R).astype(np.float32)
        best = T.viterbi_codes(v, cb)
        got = T.path_cost(v, cb, best)
        # every one of the 4^8 sequences, in the same fp32 arithmetic
        seqs = np.array(list(itertools.product(range(4), repeat=R)), dtype=np.int64)
        idx = np.zeros(len(seqs), dtype=np.int64)
        cost = np.zeros(len(seqs), dtype=np.float32)
        cbf = cb.astype(np.float32)
        for i in range(R):
            idx = (idx >> 2) | (seqs[:, i] << 14)
            d = (v[i] - cbf[idx]).astype(np.float32)
            cost = (cost + (d * d).astype(np.float32)).astype(np.float32)
        assert got == cost.min(), (trial, got, cost.min())


def test_viterbi_never_worse_than_greedy_and_exact_when_possible():
    rs = np.random.default_rng(3)
    cb = _codebook(8)
    v = (rs.standard_normal(64)).astype(np.float32)
    vit = T.path_cost(v, cb, T.viterbi_codes(v, cb))
    # greedy: each code chosen on its own, given the ones before it
    g, cur = [], 0
    cbf = cb.astype(np.float32)
    for vi in v:
        errs = [(vi - cbf[(cur >> 2) | (c << 14)]) ** 2 for c in range(4)]
        c = int(np.argmin(errs))
        g.append(c)
        cur = (cur >> 2) | (c << 14)
    assert vit <= T.path_cost(v, cb, np.array(g))
    # a codebook of +-1 and weights +-s laid out by some code sequence: a
    # zero-error path exists, so the reconstruction is exact
    cb1 = np.where(rs.random(65536) < 0.5, -1.0, 1.0).astype(np.float16)
    s = np.float16(0.03125)
    c_true = rs.integers(0, 4, 128)
    w = (cb1.astype(np.float64)[T.trellis_indices(c_true)] * float(s)).astype(np.float16)[None, :]
    codes, scales = T.pack_trellis(w, cb1)
    assert scales[0] == s
    assert np.array_equal(T.dequant_trellis(codes, scales, cb1), w.astype(np.float64))


def test_scale_closed_forms_and_zero_column():
    rs = np.random.default_rng(4)
    col = (rs.choice([-1.0, 1.0], 128) * 0.5).astype(np.float16)
    assert float(T.trellis_scale(col)) == 0.5
    col = np.array([3.0, 4.0] * 64, dtype=np.float16)      # rms = sqrt(12.5)
    assert float(T.trellis_scale(col)) == float(np.float16(np.sqrt(12.5)))
    W = WL.weights_fp16(61, 0, "w", 256, 3, 0.02)
    for j in range(3):
        s = float(T.trellis_scale(W[j]))
        true = np.sqrt((W[j].astype(np.float64) ** 2).mean())
        assert abs(s - true) <= true * 2.0 ** -11 * 1.0001
    codes, scales = T.pack_trellis(np.zeros((2, 128), dtype=np.float16), _codebook())
    assert not np.any(codes) and not np.any(scales.astype(np.float64))


def test_trellis_beats_the_scalar_code_at_two_bits():
    # section 6: trellis coding leaves less error than the scalar code at the
    # same two-bit rate
    import oracle as O
    cb = _codebook(9)
    W = WL.weights_fp16(62, 0, "w", 256, 4, 0.02)
    w = W.astype(np.float64)
    c, s = T.pack_trellis(W, cb)
    et = ((w - T.dequant_trellis(c, s, cb)) ** 2).sum()
    c2, s2 = O.pack_sign2(W)
    es = ((w - O.dequant_sign2(c2, s2)) ** 2).sum()
    assert et < 0.75 * es


def test_library_host_encoder_matches_the_oracle():
    """spax_pack_trellis_host (the library's offline encoder, host code) against
    the oracle: codes and scales bit for bit, zero and outlier columns
    included."""
    import activation_sparse_decode_token_amd as spax
    cb = _codebook(10)
    W = WL.weights_fp16(63, 0, "w", 256, 5, 0.02)
    W[1] = 0
    W[2, 7] = np.float16(3.0)
    W[3] = (np.random.default_rng(6).integers(-9, 10, 256) * 2.0 ** -24).astype(np.float16)
    codes = np.zeros((5, 64), dtype=np.uint8)
    scales = np.zeros(5, dtype=np.float16)
    spax.pack_trellis_host(W, 256, 5, cb, codes, scales, threads=3)
    oc, os_ = T.pack_trellis(W, cb)
    assert np.array_equal(scales.view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(codes, oc)
    # columns are handed out one at a time: any thread count gives the same
    for th in (1, 8):
        c2 = np.zeros_like(codes)
        s2 = np.zeros_like(scales)
        spax.pack_trellis_host(W, 256, 5, cb, c2, s2, threads=th)
        assert np.array_equal(c2, codes) and np.array_equal(s2.view(np.uint16), scales.view(np.uint16))
