"""Plain CPU oracle of the SpAx page's trellis-coded middle tier (section 5.1,
the bitshift trellis with Viterbi encoding; Figure 3).

TEST INFRASTRUCTURE, like spax_oracle. Parity status: pinned on the CPU
(brute force, closed forms); the library's GPU and host encoders and its
trellis product are checked against it in the GPU tests.

What the page fixes: per column, 2-bit codes and one scale (the column's
root-mean-square); a shared codebook of 2^16 values drawn once from a
standard normal distribution; weight i is read through the window of the
codes of rows i-7..i, a 16-bit index, times the scale; codes before the
column start are zero; the codes minimise the total squared error between
the normalised weights and their reconstructions (Viterbi).

Readings (the page leaves them open):
  * Window bits: index_i = sum_t c_{i-7+t} 4^t (the oldest code in the low
    bits), so index_i = (index_{i-1} >> 2) | (c_i << 14): moving down a row
    drops the oldest code and shifts the newest in.
  * The codebook is an input (seeded draws rounded to fp16, made by the
    workloads module): random numbers the method draws are passed in.
  * Scale: s = fp16(sqrt(S / R) 2^-24) with S = sum of w_i^2 in units of
    2^-48 (an exact integer); S / R is taken as fp64(fp64(S) / R), then one
    correctly rounded square root, then one rounding to fp16.
  * Error arithmetic in fp32, every operation rounded, no fused
    multiply-add: v_i = fp32(w_i / s) (the quotient in fp64), d = v_i - cb,
    e = d * d, cost' = cost + e. The trellis state after row i is index_i >> 2
    (the last 7 codes); state t at row i is reached from state
    ((t & 0xFFF) << 2) | o of row i-1 through index 4t + o, and keeps the
    smallest cost, the smallest o on ties. Start: state 0 (zero codes) at
    cost 0, every other state unreachable. End: the smallest final cost, the
    smallest state on ties, traced back.
  * Storage: the int2 packing (row 4i + r in bits 2r..2r+1 of byte i) and
    one fp16 scale per column. A zero column gets scale 0 and zero codes.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .spax_oracle import fp16_round

__all__ = ["trellis_scale", "trellis_indices", "viterbi_codes", "pack_trellis",
           "dequant_trellis", "path_cost"]

N_STATES = 1 << 14


def trellis_scale(col: np.ndarray) -> np.float16:
    """fp16 root-mean-square of a column (exact sum of squares)."""
    w = [int(v) for v in (np.asarray(col, dtype=np.float16).astype(np.float64)
                          * 2.0 ** 24).astype(np.int64)]
    S = sum(v * v for v in w)                       # units of 2^-48, exact
    q = float(S) / float(len(w))
    return fp16_round(np.sqrt(q) * 2.0 ** -24)[()]


def trellis_indices(codes_seq: np.ndarray) -> np.ndarray:
    """index_i = (index_{i-1} >> 2) | (c_i << 14), index_{-1} = 0."""
    idx = np.empty(len(codes_seq), dtype=np.int64)
    cur = 0
    for i, c in enumerate(codes_seq):
        cur = (cur >> 2) | (int(c) << 14)
        idx[i] = cur
    return idx


def path_cost(v: np.ndarray, cb: np.ndarray, codes_seq: np.ndarray) -> np.float32:
    """The fp32 cost of one code sequence, summed in row order."""
    cbf = np.asarray(cb, dtype=np.float16).astype(np.float32)
    cost = np.float32(0.0)
    for vi, k in zip(np.asarray(v, dtype=np.float32), trellis_indices(codes_seq)):
        d = np.float32(vi - cbf[k])
        cost = np.float32(cost + np.float32(d * d))
    return cost


def viterbi_codes(v: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """The code sequence of least fp32 cost (the tie rules above)."""
    v = np.asarray(v, dtype=np.float32)
    cbf = np.asarray(cb, dtype=np.float16).astype(np.float32)
    R = len(v)
    t = np.arange(N_STATES, dtype=np.int64)
    pred = ((t & 0xFFF) << 2)[:, None] | np.arange(4, dtype=np.int64)[None, :]   # [T, 4]
    win = (4 * t)[:, None] + np.arange(4, dtype=np.int64)[None, :]               # [T, 4]
    cost = np.full(N_STATES, np.inf, dtype=np.float32)
    cost[0] = 0.0
    back = np.empty((R, N_STATES), dtype=np.uint8)
    with np.errstate(invalid="ignore", over="ignore"):
        for i in range(R):
            d = (v[i] - cbf[win]).astype(np.float32)
            cand = (cost[pred] + (d * d).astype(np.float32)).astype(np.float32)
            o = np.argmin(cand, axis=1)                  # first minimum: smallest o
            back[i] = o
            cost = cand[t, o]
    state = int(np.argmin(cost))                         # smallest state on ties
    codes = np.empty(R, dtype=np.int64)
    for i in range(R - 1, -1, -1):
        codes[i] = state >> 12
        state = ((state & 0xFFF) << 2) | int(back[i, state])
    return codes


def pack_trellis(Wt: np.ndarray, cb: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Codes uint8 [n, R/4] (int2 packing) and scales fp16 [n] of each column."""
    n, R = Wt.shape
    if R % 4:
        raise ValueError("rows must be a multiple of 4")
    codes = np.zeros((n, R // 4), dtype=np.uint8)
    scales = np.zeros(n, dtype=np.float16)
    for j in range(n):
        s = trellis_scale(Wt[j])
        scales[j] = s
        if float(s) == 0.0:
            continue
        v = (Wt[j].astype(np.float64) / float(s)).astype(np.float32)
        c = viterbi_codes(v, cb)
        codes[j] = (c[0::4] | (c[1::4] << 2) | (c[2::4] << 4) | (c[3::4] << 6)).astype(np.uint8)
    return codes, scales


def dequant_trellis(codes: np.ndarray, scales: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """w_hat_i = cb[index_i] * s in fp64 (exact); returns [n, R]."""
    n = codes.shape[0]
    R = codes.shape[1] * 4
    cbd = np.asarray(cb, dtype=np.float16).astype(np.float64)
    out = np.empty((n, R), dtype=np.float64)
    for j in range(n):
        c = np.empty(R, dtype=np.int64)
        for r in range(4):
            c[r::4] = (codes[j] >> (2 * r)) & 3
        out[j] = cbd[trellis_indices(c)] * float(scales[j])
    return out
