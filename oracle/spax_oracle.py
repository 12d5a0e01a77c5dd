"""Plain, slow CPU oracle for SpAx-style three-tier activation sparsity.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import this module. It shares no code with the HIP
library and imports nothing from it.

Source: the SpAx page, "Activation Sparsity with Weight Approximation for
Faster LLM Decoding on Offloaded Weights".
Each function names the section, equation or figure it follows.

Everything is written as the plain definition:
  * tier selection is a stable sort on |x| (a library sort is the one step);
  * packing is exact fp64 arithmetic followed by one rounding;
  * the tiered product sums exact fp64 products in fp64 (a library matmul is
    the one step) and is rounded once to fp16 by the caller's choice.

Readings of points the page leaves open (tie-break, list order, code format,
group orientation, rounding) are stated at each function below.

Storage convention: a matrix of R rows and n columns is an array of shape
[n, R] (column-major); row j of the array is column j of the matrix.

Parity status: every function here is pinned by tests/test_oracle.py against
closed forms, brute force, hand-worked golden files or exact rational
arithmetic. The fp32 summation order of the GPU is not modelled (parity
unpinned beyond the stated error bound, by design: several results are
correct).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = [
    "magnitude_key", "plan_tiers", "fp16_round",
    "pack_int4_g128", "pack_int2_g128", "dequant_int4_g128", "dequant_int2_g128",
    "pack_sign2", "dequant_sign2", "fp16_units",
    "ColumnStore", "tiered_product", "tiered_gemv_fp16",
    "silu", "swiglu_fp16", "layer_step", "GROUP_SIZE",
]

GROUP_SIZE = 128  # rows per quantisation group within one column


# --------------------------------------------------------------------------
# Tier selection -- SpAx page section 2 (magnitude top-k) and section 5,
# Figure 2 step 3 (rank by magnitude, second boundary splits the kept
# entries into top and middle tiers).
# --------------------------------------------------------------------------

def magnitude_key(x: np.ndarray) -> np.ndarray:
    """Sort key of |x_j| for fp16 inputs: the 15-bit magnitude pattern.

    For fp16 the bit pattern with the sign cleared orders the same as |x|
    (finite values, then inf, then NaN patterns above inf); +0 and -0 share
    key 0 and tie."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    return (x.view(np.uint16) & np.uint16(0x7FFF)).astype(np.int64)


def plan_tiers(x: np.ndarray, k_full: int, k_approx: int) -> Tuple[np.ndarray, np.ndarray]:
    """Split the columns of one projection into full / approx / skip tiers.

    SpAx page section 5, Figure 2 step 3 and section 5.2: rank the input
    activations by magnitude; the k_top largest select full-precision
    columns, the next k_mid select compressed columns, the rest are skipped.

    Readings: equal magnitudes rank the lower index first (a stable sort on
    descending key); both lists are returned in ascending index order.

    Returns (full_idx, approx_idx) as int32 arrays.
    """
    key = magnitude_key(x)
    n = key.shape[0]
    if k_full < 0 or k_approx < 0 or k_full + k_approx > n:
        raise ValueError("need 0 <= k_full, 0 <= k_approx, k_full + k_approx <= n")
    # stable sort on (-key): descending magnitude, ascending index among ties
    order = np.argsort(-key, kind="stable")
    full = np.sort(order[:k_full]).astype(np.int32)
    approx = np.sort(order[k_full:k_full + k_approx]).astype(np.int32)
    return full, approx


# --------------------------------------------------------------------------
# fp16 rounding (round to nearest, ties to even) of fp64 values.
# --------------------------------------------------------------------------

def fp16_round(v) -> np.ndarray:
    """Round float64 values to the nearest fp16 value, ties to even.

    numpy's float64 -> float16 cast rounds once, directly from the double;
    tests/test_oracle.py pins it against exact rational rounding."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


# --------------------------------------------------------------------------
# Middle-tier code. SpAx page section 5.1: each column is encoded on its own
# so that a selected column can be rebuilt from its own codes and scales;
# Eq. 4 reconstructs a weight as a sum of signed per-column scales.
# The format here is the group-128 integer code with fp16 scales: groups are
# 128 consecutive rows of one column (keeps columns independent).
# --------------------------------------------------------------------------

def _groups(Wt: np.ndarray) -> np.ndarray:
    n, R = Wt.shape
    if R % GROUP_SIZE:
        raise ValueError("rows must be a multiple of 128")
    return Wt.astype(np.float64).reshape(n, R // GROUP_SIZE, GROUP_SIZE)


def pack_int4_g128(Wt: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int4 code per 128-row group of each column.

    For each group with m = max |w|:
        s = fp16(m / 7)                       (one rounding of the quotient)
        q = clamp(round_half_even(w / s), -8, 7)   (q = 0 when s == 0)
        w_hat = q * s
    Row 2i is stored in bits 0-3 of byte i of the column, row 2i+1 in bits
    4-7, as a two's-complement nibble.

    Wt: fp16 [n, R]. Returns codes uint8 [n, R/2] and scales fp16 [n, R/128].
    """
    n, R = Wt.shape
    w = _groups(Wt)
    m = np.abs(w).max(axis=2)
    s = fp16_round(m / 7.0)
    s64 = s.astype(np.float64)[..., None]
    q = np.zeros_like(w)
    nz = np.broadcast_to(s64 > 0, w.shape)
    q[nz] = np.rint(w[nz] / np.broadcast_to(s64, w.shape)[nz])
    q = np.clip(q, -8, 7).astype(np.int64).reshape(n, R)
    nib = (q & 0xF).astype(np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, s


def dequant_int4_g128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w_hat = q * s in fp64 for int4 codes; returns [n, R]."""
    n = codes.shape[0]
    R = codes.shape[1] * 2
    nib = np.empty((n, R), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    q = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    s = np.repeat(scales.astype(np.float64), GROUP_SIZE, axis=1)
    return q * s


def pack_int2_g128(Wt: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Four-level mid-rise int2 code per 128-row group of each column.

    The levels are +-0.5 s and +-1.5 s: the SpAx page's two-scale form
    w_hat = e1 s0 + e2 s1 with e in {-1, +1} (section 5.1, Eq. 4), taken with
    s0 = s, s1 = s / 2 and one fp16 scale per group. With m = max |w|:
        s = fp16(m / 1.5)
        u = clamp(round_half_even(w / s + 1.5), 0, 3)   (u = 2 when s == 0)
        w_hat = (u - 1.5) * s
    Row 4i + r is stored in bits 2r..2r+1 of byte i of the column.

    Returns codes uint8 [n, R/4] and scales fp16 [n, R/128].
    """
    n, R = Wt.shape
    w = _groups(Wt)
    m = np.abs(w).max(axis=2)
    s = fp16_round(m / 1.5)
    s64 = s.astype(np.float64)[..., None]
    u = np.full_like(w, 2.0)
    nz = np.broadcast_to(s64 > 0, w.shape)
    u[nz] = np.rint(w[nz] / np.broadcast_to(s64, w.shape)[nz] + 1.5)
    u = np.clip(u, 0, 3).astype(np.int64).reshape(n, R)
    codes = (u[:, 0::4] | (u[:, 1::4] << 2) | (u[:, 2::4] << 4) | (u[:, 3::4] << 6))
    return codes.astype(np.uint8), s


def dequant_int2_g128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w_hat = (u - 1.5) * s in fp64 for int2 codes; returns [n, R]."""
    n = codes.shape[0]
    R = codes.shape[1] * 4
    u = np.empty((n, R), dtype=np.int64)
    for r in range(4):
        u[:, r::4] = (codes >> (2 * r)) & 3
    s = np.repeat(scales.astype(np.float64), GROUP_SIZE, axis=1)
    return (u.astype(np.float64) - 1.5) * s


# --------------------------------------------------------------------------
# The SpAx page's own scalar middle-tier code (section 5.1, Eq. 4): every
# weight of column j is rebuilt as e1 s_{j,0} + e2 s_{j,1} with two sign
# codes (e1, e2) in {-1, +1} and two scales per column; the codes are the
# argmin of the squared error given the scales.
# --------------------------------------------------------------------------

def fp16_units(Wt: np.ndarray) -> np.ndarray:
    """fp16 values as exact integers in units of 2^-24 (every finite fp16
    value is a multiple of 2^-24 below 2^16, so |w| 2^24 < 2^40)."""
    return (np.asarray(Wt, dtype=np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)


def _mean_to_fp16(total: np.ndarray, count: int) -> np.ndarray:
    """fp16(total 2^-24 / count) for exact integer totals: one fp64 division
    of the two (exact) operands, then one rounding to fp16."""
    return fp16_round(total.astype(np.float64) / float(count) * 2.0 ** -24)


def pack_sign2(Wt: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Two-scale 2-bit sign code of each column (SpAx page section 5.1, Eq. 4).

    Scales (the page fits them Lloyd-Max style; the fitting text is lost, so
    the reading here is the closed-form greedy fit, each scale the
    least-squares optimum for its own sign code):
        e1_i = +1 if w_i >= 0 else -1
        s0 = fp16(mean_i |w_i|)
        s1 = fp16(mean_i |w_i - e1_i s0|)
    Codes: (e1, e2) = argmin over {-1, +1}^2 of (w_i - e1 s0 - e2 s1)^2 with
    the stored (fp16) scales; among equal errors the smaller code u wins.
    The 2-bit code is u = 2 [e1 = -1] + [e2 = -1]; row 4i + r is stored in
    bits 2r..2r+1 of byte i of the column (the int2 packing).
    All arithmetic is exact: weights and scales as integers in units of
    2^-24, so sums and distances never round; the two means are rounded
    once each (fp64 division, then fp16).

    Wt: fp16 [n, R]. Returns codes uint8 [n, R/4] and scales fp16 [n, 2]
    (s0, s1)."""
    n, R = Wt.shape
    if R % 4:
        raise ValueError("rows must be a multiple of 4")
    w = fp16_units(Wt)                                   # exact, signed
    s0 = _mean_to_fp16(np.abs(w).sum(axis=1), R)
    s0u = fp16_units(s0)[:, None]
    e1 = np.where(w >= 0, 1, -1)
    s1 = _mean_to_fp16(np.abs(w - e1 * s0u).sum(axis=1), R)
    s1u = fp16_units(s1)[:, None]
    # candidate levels in code order u = 0..3: (+,+), (+,-), (-,+), (-,-)
    levels = [s0u + s1u, s0u - s1u, -s0u + s1u, -s0u - s1u]
    dist = np.stack([np.abs(w - L) for L in levels])     # [4, n, R], exact
    u = np.argmin(dist, axis=0).astype(np.int64)         # first minimum: smallest u
    codes = (u[:, 0::4] | (u[:, 1::4] << 2) | (u[:, 2::4] << 4) | (u[:, 3::4] << 6))
    scales = np.stack([s0, s1], axis=1).astype(np.float16)
    return codes.astype(np.uint8), scales


def dequant_sign2(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w_hat = e1 s0 + e2 s1 in fp64 (exact); returns [n, R]."""
    n = codes.shape[0]
    R = codes.shape[1] * 4
    u = np.empty((n, R), dtype=np.int64)
    for r in range(4):
        u[:, r::4] = (codes >> (2 * r)) & 3
    e1 = np.where(u & 2, -1.0, 1.0)
    e2 = np.where(u & 1, -1.0, 1.0)
    s = scales.astype(np.float64)
    return e1 * s[:, 0:1] + e2 * s[:, 1:2]


class ColumnStore:
    """One tier's copy of a matrix: fp16 columns, or int4 / int2 / sign2 codes.

    columns(idx) returns the exact fp64 values of the selected columns as an
    array [len(idx), R] (SpAx page, Figure 2 step 5: the GPU rebuilds the
    compressed columns from their codes)."""

    def __init__(self, fmt: str, Wt: Optional[np.ndarray] = None,
                 codes: Optional[np.ndarray] = None, scales: Optional[np.ndarray] = None):
        self.fmt = fmt
        if fmt == "fp16":
            self.Wt = np.ascontiguousarray(Wt, dtype=np.float16)
            self.rows = self.Wt.shape[1]
        elif fmt in ("int4", "int2", "sign2"):
            if codes is None:
                codes, scales = {"int4": pack_int4_g128, "int2": pack_int2_g128,
                                 "sign2": pack_sign2}[fmt](Wt)
            self.codes, self.scales = codes, scales
            self.rows = codes.shape[1] * (2 if fmt == "int4" else 4)
        else:
            raise ValueError(fmt)

    def columns(self, idx: np.ndarray) -> np.ndarray:
        idx = np.asarray(idx, dtype=np.int64)
        if self.fmt == "fp16":
            return self.Wt[idx].astype(np.float64)
        if self.fmt == "int4":
            return dequant_int4_g128(self.codes[idx], self.scales[idx])
        if self.fmt == "sign2":
            return dequant_sign2(self.codes[idx], self.scales[idx])
        return dequant_int2_g128(self.codes[idx], self.scales[idx])


# --------------------------------------------------------------------------
# Tiered product -- SpAx page section 2 Eq. 1 (a projection with skipped
# entries is the sum of the kept columns scaled by their activations) and
# section 5, Figure 2 steps 4-5 (full columns plus rebuilt middle columns).
# --------------------------------------------------------------------------

def tiered_product(x: np.ndarray, full_idx: np.ndarray, approx_idx: np.ndarray,
                   full: ColumnStore, approx: Optional[ColumnStore]) -> np.ndarray:
    """r = sum_{j in F} x_j W~[:, j] + sum_{j in A} x_j W^[:, j] in fp64.

    Each product of an fp16 activation with an fp16 weight or a dequantised
    code is exact in fp64; the sums are taken in fp64."""
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    r = np.zeros(full.rows, dtype=np.float64)
    if len(full_idx):
        r += xf[full_idx] @ full.columns(full_idx)
    if len(approx_idx):
        if approx is None:
            raise ValueError("approx indices given without an approx copy")
        r += xf[approx_idx] @ approx.columns(approx_idx)
    return r


def tiered_gemv_fp16(x, full_idx, approx_idx, full, approx) -> np.ndarray:
    """The tiered product rounded once to fp16 (the library's output type)."""
    return fp16_round(tiered_product(x, full_idx, approx_idx, full, approx))


# --------------------------------------------------------------------------
# SwiGLU -- SpAx page section 2: a = sigma(W_gate x) (.) W_up x with sigma =
# SiLU, applied to the fp16 outputs of the gate and up projections.
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_fp16(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """a = fp16(silu(g) * u) for fp16 g, u."""
    g64 = np.asarray(g, dtype=np.float16).astype(np.float64)
    u64 = np.asarray(u, dtype=np.float16).astype(np.float64)
    return fp16_round(silu(g64) * u64)


# --------------------------------------------------------------------------
# One decoder layer's projections -- SpAx page section 2 (the seven matrices
# and their inputs) and sections 5.2 / 5.3 (four groups that share one
# ranking: (q, k, v) on h, (o) on z, (gate, up) on x, (down) on a).
# --------------------------------------------------------------------------

def layer_step(mats: dict, ks: dict, h=None, z=None, x=None) -> dict:
    """Run the four ranking groups of one layer.

    mats: name -> (full ColumnStore, approx ColumnStore or None) for any of
          q, k, v, o, gate, up, down.
    ks:   group -> (k_full, k_approx) for groups "qkv", "o", "ffn", "down".
    Inputs h, z, x are fp16 vectors; a is computed from gate and up.
    Returns fp16 outputs and the tier lists of every group that ran.
    """
    out = {}
    if h is not None and "q" in mats:
        F, A = plan_tiers(h, *ks["qkv"])
        out["qkv_lists"] = (F, A)
        for name in ("q", "k", "v"):
            out[name] = tiered_gemv_fp16(h, F, A, *mats[name])
    if z is not None and "o" in mats:
        F, A = plan_tiers(z, *ks["o"])
        out["o_lists"] = (F, A)
        out["o"] = tiered_gemv_fp16(z, F, A, *mats["o"])
    if x is not None and "gate" in mats:
        F, A = plan_tiers(x, *ks["ffn"])
        out["ffn_lists"] = (F, A)
        g = tiered_gemv_fp16(x, F, A, *mats["gate"])
        u = tiered_gemv_fp16(x, F, A, *mats["up"])
        out["g"], out["u"] = g, u
        out["a"] = swiglu_fp16(g, u)
        F2, A2 = plan_tiers(out["a"], *ks["down"])
        out["down_lists"] = (F2, A2)
        out["down"] = tiered_gemv_fp16(out["a"], F2, A2, *mats["down"])
    return out

