"""Byte and roofline accounting for the benchmark (measurement definitions).

No part of the method is computed here; these functions count the bytes the
method must move and turn them into bandwidth floors.

* Read budget (SpAx page, section 5.2 Eq. 5, and section 6 setup): the weight
  data needed per token -- selected original columns, compressed codes and
  any auxiliary data such as scales -- over the dense size of the same
  matrices: budget = (k_top + rho * k_mid) / n, rho = middle-tier bytes per
  column / full-tier bytes per column.
* Decode roofline (LazyWeights explainer page, the roofline and the worked
  example): a decode projection moves about one flop per byte, so its time is
  at least bytes / bandwidth; a decoder of coded weights must run at
  theta* = 8 beta / b_c weights per second to keep pace with bandwidth beta.
"""
from __future__ import annotations

GROUP = 128


def column_bytes(fmt: str, rows: int) -> int:
    """Bytes of one stored column: fp16 values, or codes plus fp16 scales."""
    if fmt == "fp16":
        return 2 * rows
    if fmt == "int4":
        return rows // 2 + 2 * (rows // GROUP)
    if fmt == "int2":
        return rows // 4 + 2 * (rows // GROUP)
    if fmt == "sign2":                      # 2-bit codes and two fp16 scales
        return rows // 4 + 4
    if fmt == "trellis":                    # 2-bit codes and one fp16 scale
        return rows // 4 + 2
    if fmt == "none":
        return 0
    raise ValueError(fmt)


def gemv_algorithmic_bytes(rows: int, n: int, k_full: int, k_approx: int,
                           full_fmt: str, approx_fmt: str) -> int:
    """Bytes one tiered projection must move: the selected full columns, the
    selected code columns with their scales, the input x (fp16), both index
    lists (int32) and the output y (fp16). Skipped columns are not counted."""
    return (k_full * column_bytes(full_fmt, rows)
            + k_approx * column_bytes(approx_fmt, rows)
            + 2 * n + 4 * (k_full + k_approx) + 2 * rows)


def rho(full_fmt: str, approx_fmt: str, rows: int) -> float:
    return column_bytes(approx_fmt, rows) / column_bytes(full_fmt, rows)


def budget(k_full: int, k_approx: int, n: int, rho_: float) -> float:
    """Eq. 5 of the SpAx page: (k_top + rho k_mid) / n."""
    return (k_full + rho_ * k_approx) / n


def floor_seconds(nbytes: float, bandwidth_bytes_per_s: float) -> float:
    """Bandwidth floor of a memory-bound pass: bytes / bandwidth."""
    return nbytes / bandwidth_bytes_per_s


def decode_rate(bandwidth_bytes_per_s: float, bits_per_weight: float) -> float:
    """theta* = 8 beta / b_c: weights per second a decoder must sustain."""
    return 8.0 * bandwidth_bytes_per_s / bits_per_weight


HBM_PEAK_BYTES_PER_S = 8.0e12      # MI355X HBM3E, published peak
PCIE5_X16_BYTES_PER_S = 64.0e9     # nominal per direction
