"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O

GROUP = 128
# Stated tolerance for fp16 outputs with fp32 accumulation: max relative error
# 2e-3, norm-wise (|y - r|_inf / |r|_inf).
REL_TOL = 2e-3
U24 = 2.0 ** -24
FP16_MIN_NORMAL = 2.0 ** -14


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def ulp16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def abs_sum(x, F, A, full: O.ColumnStore, approx) -> np.ndarray:
    """Per-row sum of the magnitudes the fp32 accumulation adds: |x_j W_ij|
    for full fp16 columns; |x_j| (s_{j,0} + s_{j,1}) for a two-scale sign
    code column (its two terms). A code column with b-bit code u adds
    x_j s_jg (2^b + u) per element (the code as fp16 1 + u / 2^b times the
    factor 2^b x_j s_jg) and x_j s_jg (2^b + offset) once to the running sum
    that is subtracted at the end (offset 8 for int4, 1.5 for int2)."""
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    S = np.zeros(full.rows)

    def code_part(store, idx):
        if hasattr(store, "abs_terms"):
            # a stored column of several matrices, each coded on its own
            return np.abs(xf[idx])[:, None] * store.abs_terms(idx)
        if store.fmt == "trellis":
            # one term per element: the codebook value times x_j s_j
            return np.abs(xf[idx])[:, None] * np.abs(store.columns(idx))
        if store.fmt == "sign2":
            # two exact terms per element: +-x_j s_{j,0} and +-x_j s_{j,1}
            s = store.scales[idx].astype(np.float64)
            return np.repeat((np.abs(xf[idx]) * (s[:, 0] + s[:, 1]))[:, None], store.rows, axis=1)
        if store.fmt == "int4":
            nib = np.empty((len(idx), store.rows), dtype=np.int64)
            c = store.codes[idx]
            nib[:, 0::2] = c & 0xF
            nib[:, 1::2] = c >> 4
            u = (nib ^ 8).astype(np.float64)
            base, off = 16.0, 8.0
        else:
            c = store.codes[idx]
            u = np.empty((len(idx), store.rows), dtype=np.float64)
            for r in range(4):
                u[:, r::4] = (c >> (2 * r)) & 3
            base, off = 4.0, 1.5
        s = np.repeat(store.scales[idx].astype(np.float64), GROUP, axis=1)
        return np.abs(xf[idx])[:, None] * s * ((base + u) + (base + off))

    if len(F):
        if full.fmt == "fp16":
            S += np.abs(xf[F]) @ np.abs(full.columns(F))
        else:
            S += code_part(full, F).sum(axis=0)
    if len(A):
        S += code_part(approx, A).sum(axis=0)
    return S


def check_product(y16: np.ndarray, x, F, A, full, approx, label: str = "",
                  rows: np.ndarray | None = None) -> float:
    """Compare a GPU fp16 output with the oracle.

    Gate: |y - r|_inf <= 2e-3 |r|_inf. Also every element must sit within
    the order-independent bound gamma_m * S_i + ulp16(y_i)/2 of the exact
    value r_i (m = terms summed, S_i = abs_sum); an all-zero r needs y == 0.
    `rows` optionally names the stored rows the stores were cut to.
    Returns the norm-wise error."""
    r = O.tiered_product(x, F, A, full, approx)
    y = np.asarray(y16, dtype=np.float16).astype(np.float64)
    if rows is not None:
        y = y[rows]
    assert y.shape == r.shape
    rmax = np.abs(r).max() if r.size else 0.0
    if rmax == 0.0:
        assert np.all(y == 0), f"{label}: expected zeros"
        return 0.0
    err = np.abs(y - r).max() / rmax
    # Below the smallest normal fp16 (2^-14) the output grid is an absolute
    # 2^-24, so a relative gate cannot hold for any rounding; there the
    # elementwise bound below is the gate.
    if rmax >= FP16_MIN_NORMAL:
        assert err <= REL_TOL, f"{label}: norm-wise error {err:.3e} > {REL_TOL}"
    # terms summed per element: one per full or integer-code column, two per
    # sign-code column, plus the split partials and the running offset sum
    per_a = 2 if approx is not None and approx.fmt == "sign2" else 1
    m = len(F) + per_a * len(A) + 80
    gamma = m * U24 / (1 - m * U24)
    S = abs_sum(x, F, A, full, approx)
    bound = gamma * S + 0.5 * ulp16(y) + 2.0 ** -25
    bad = np.abs(y - r) > bound
    assert not bad.any(), (f"{label}: {bad.sum()} elements outside the fp32 bound, "
                           f"first at {np.argmax(bad)}")
    return float(err)


def sample_groups(R: int, n_groups: int, seed: int) -> np.ndarray:
    """Stored rows of a few whole 128-row groups: the first, the last, both
    sides of every 512-row tile boundary near the start, and random ones."""
    G = R // GROUP
    rs = np.random.default_rng(seed)
    pick = {0, G - 1, min(3, G - 1), min(4, G - 1)}
    pick |= set(rs.choice(G, size=min(n_groups, G), replace=False).tolist())
    g = np.array(sorted(pick))
    return (g[:, None] * GROUP + np.arange(GROUP)[None, :]).ravel()


class TrellisStore:
    """Oracle view of a trellis-coded copy (codes, scales, codebook): the
    columns are the oracle's reconstruction cb[index_i] s_j."""
    fmt = "trellis"

    def __init__(self, codes: np.ndarray, scales: np.ndarray, cb: np.ndarray):
        self.codes, self.scales, self.cb = codes, scales, cb
        self.rows = codes.shape[1] * 4

    def columns(self, idx):
        from oracle.spax_trellis import dequant_trellis
        idx = np.asarray(idx, dtype=np.int64)
        return dequant_trellis(self.codes[idx], self.scales[idx], self.cb)


class RowsOf:
    """Some rows of a store whose columns are rebuilt whole (the scales and
    the trellis window run down the whole matrix column)."""

    def __init__(self, inner, rows):
        self.inner, self.rows_idx = inner, np.asarray(rows)
        self.fmt, self.rows = inner.fmt, len(self.rows_idx)
        if hasattr(inner, "abs_terms"):
            self.abs_terms = lambda idx: inner.abs_terms(idx)[:, self.rows_idx]
        elif inner.fmt == "sign2":
            self.abs_terms = lambda idx: np.repeat(
                inner.scales[np.asarray(idx)].astype(np.float64).sum(axis=1)[:, None],
                inner.rows, axis=1)[:, self.rows_idx]

    def columns(self, idx):
        return self.inner.columns(idx)[:, self.rows_idx]


class SegmentedStore:
    """Oracle view of a stored column that holds several matrices' columns,
    each coded on its own (SpAx page section 5.1): q, k, v stacked, or gate
    and up interleaved in 128-row blocks ("glu"). columns(idx) puts each
    matrix's rebuilt columns at its stored rows; abs_terms(idx) gives the
    magnitude the kernel adds per element and unit |x_j| (the sign code: its
    matrix's s0 + s1; the trellis code: |value|)."""

    def __init__(self, stores, layout: str = "stacked"):
        self.stores, self.layout = list(stores), layout
        self.fmt = self.stores[0].fmt
        self.rows = sum(st.rows for st in self.stores)

    def _place(self, parts):
        if self.layout == "glu":
            g, u = parts
            k, I = g.shape
            out = np.empty((k, 2 * I), dtype=np.float64)
            v = out.reshape(k, I // GROUP, 2, GROUP)
            v[:, :, 0, :] = g.reshape(k, I // GROUP, GROUP)
            v[:, :, 1, :] = u.reshape(k, I // GROUP, GROUP)
            return out
        return np.concatenate(parts, axis=1)

    def columns(self, idx):
        return self._place([st.columns(idx) for st in self.stores])

    def abs_terms(self, idx):
        idx = np.asarray(idx, dtype=np.int64)
        if self.fmt == "sign2":
            parts = [np.repeat(st.scales[idx].astype(np.float64).sum(axis=1)[:, None], st.rows,
                               axis=1) for st in self.stores]
        else:
            parts = [np.abs(st.columns(idx)) for st in self.stores]
        return self._place(parts)


def split_codes(codes: np.ndarray, scales: np.ndarray, n_mat: int, layout: str = "stacked"):
    """Per-matrix (codes, scales) of a stored 2-bit code (4 rows per byte) whose
    columns hold n_mat matrices: stacked row segments, or ("glu") gate and up
    in 128-row (32-byte) blocks; scales [n, n_mat * k] -> [n, k] each."""
    n, b = codes.shape
    if layout == "glu":
        v = codes.reshape(n, b // 64, 2, 32)
        parts = [np.ascontiguousarray(v[:, :, m, :].reshape(n, b // 2)) for m in range(2)]
    else:
        parts = [np.ascontiguousarray(c) for c in np.split(codes, n_mat, axis=1)]
    k = scales.shape[1] // n_mat
    sc = [np.ascontiguousarray(scales[:, m * k:(m + 1) * k]) for m in range(n_mat)]
    return [(p, s_ if k > 1 else s_[:, 0]) for p, s_ in zip(parts, sc)]
