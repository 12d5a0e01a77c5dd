"""Offline weight preparation for the library's storage layouts.

Weights are column-major: a matrix of R rows and n columns is a tensor of
shape [n, R] whose row j is column j (contiguous). Matrices that share an
input are stored as one matrix so that the columns one activation entry
indexes are adjacent (SpAx page, section 5.3, Figure 4):
  * q, k, v: rows stacked, column j = [q_j; k_j; v_j];
  * gate, up: rows interleaved in 128-row blocks (SPAX_LAYOUT_GLU_INTERLEAVED).
The compressed copies are produced by the library's packers (spax_pack_g128,
spax_pack_sign2, spax_pack_trellis). The sign and trellis codes carry
per-column scales and (trellis) a window over the column's earlier rows, so
a stored column that holds several matrices' columns is coded matrix by
matrix (SpAx page section 5.1: codes and scales per weight column; section
5.3: stacked columns stay distinct columns): each matrix is packed on its
own and its codes are placed at its rows, its scales side by side.
These helpers only move data; nothing here is on the per-token path.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (FMT_FP16, FMT_INT2_G128, FMT_INT4_G128, FMT_NONE, FMT_SIGN2, FMT_TRELLIS,
               LAYOUT_GLU_INTERLEAVED, LAYOUT_PLAIN, RES_DEVICE, RES_HOST_PINNED, Matrix,
               pack_g128, pack_sign2, pack_trellis, pack_trellis_host,
               pack_trellis_workspace_bytes)

GROUP = 128


def stack_rows(cols_major: Sequence[torch.Tensor]) -> torch.Tensor:
    """[n, R_i] tensors -> [n, sum R_i]: column j holds every matrix's column j."""
    return torch.cat(list(cols_major), dim=1).contiguous()


def glu_interleave(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """[n, I] gate and up -> [n, 2I] interleaved in 128-row blocks."""
    n, I = gate.shape
    if up.shape != gate.shape or I % GROUP:
        raise ValueError("gate and up must share a shape with I % 128 == 0")
    g = gate.reshape(n, I // GROUP, 1, GROUP)
    u = up.reshape(n, I // GROUP, 1, GROUP)
    return torch.cat([g, u], dim=2).reshape(n, 2 * I).contiguous()


def glu_deinterleave(stacked: torch.Tensor):
    """Inverse of glu_interleave along the last dimension (rows)."""
    *lead, R2 = stacked.shape
    v = stacked.reshape(*lead, R2 // (2 * GROUP), 2, GROUP)
    return v[..., 0, :].reshape(*lead, R2 // 2), v[..., 1, :].reshape(*lead, R2 // 2)


# Largest backpointer workspace the GPU trellis encoder may take (columns are
# encoded in launches of as many columns as fit; 4 KB per row per column).
TRELLIS_WS_BYTES = 1 << 31


def pack(w_cm: torch.Tensor, fmt: int, stream=None, codebook: Optional[torch.Tensor] = None,
         trellis_on_host: bool = False, trellis_ws_bytes: Optional[int] = None):
    """Codes and scales of a column-major fp16 device tensor [n, R]. The
    trellis code uses the given device codebook (fp16 [65536]) and is encoded
    on the GPU (spax_pack_trellis, a backpointer workspace of up to
    trellis_ws_bytes) or, with trellis_on_host, by the host encoder
    (spax_pack_trellis_host); both give the same bits."""
    n, R = w_cm.shape
    if fmt == FMT_TRELLIS:
        import numpy as np
        if codebook is None:
            raise ValueError("the trellis code needs a codebook")
        if trellis_on_host:
            w_h = w_cm.detach().cpu().contiguous().numpy()
            cb_h = codebook.detach().cpu().contiguous().numpy()
            codes = np.zeros((n, R // 4), dtype=np.uint8)
            scales = np.zeros(n, dtype=np.float16)
            pack_trellis_host(w_h, R, n, cb_h, codes, scales)
            return (torch.from_numpy(codes).to(w_cm.device),
                    torch.from_numpy(scales).to(w_cm.device))
        codes = torch.empty((n, R // 4), dtype=torch.uint8, device=w_cm.device)
        scales = torch.empty(n, dtype=torch.float16, device=w_cm.device)
        per = pack_trellis_workspace_bytes(R, 1)
        cap = TRELLIS_WS_BYTES if trellis_ws_bytes is None else trellis_ws_bytes
        ws = torch.empty(max(per, min(cap, per * n)), dtype=torch.uint8, device=w_cm.device)
        pack_trellis(w_cm, R, n, codebook, codes, scales, ws, stream=stream)
        return codes, scales
    if fmt == FMT_SIGN2:
        # two-scale sign code: 2 bits per weight, (s0, s1) per column
        codes = torch.empty((n, R // 4), dtype=torch.uint8, device=w_cm.device)
        scales = torch.empty((n, 2), dtype=torch.float16, device=w_cm.device)
        pack_sign2(w_cm, R, n, codes, scales, stream)
        return codes, scales
    per = {FMT_INT4_G128: 2, FMT_INT2_G128: 4}[fmt]
    codes = torch.empty((n, R // per), dtype=torch.uint8, device=w_cm.device)
    scales = torch.empty((n, R // GROUP), dtype=torch.float16, device=w_cm.device)
    pack_g128(w_cm, R, n, fmt, codes, scales, stream)
    return codes, scales


def _segments(w_cm: torch.Tensor, layout: int, seg_rows: int):
    """The matrices of a stored column-major tensor [n, R]: gate and up of
    the GLU layout, or the stacked segments of seg_rows rows (one when 0)."""
    if layout == LAYOUT_GLU_INTERLEAVED:
        return [t.contiguous() for t in glu_deinterleave(w_cm)]
    if seg_rows:
        return [t.contiguous() for t in w_cm.split(seg_rows, dim=1)]
    return [w_cm]


def pack_per_matrix(w_cm: torch.Tensor, fmt: int, layout: int = LAYOUT_PLAIN,
                    seg_rows: int = 0, stream=None, codebook: Optional[torch.Tensor] = None,
                    **kw):
    """Sign or trellis codes and scales of a stored tensor whose columns hold
    several matrices' columns, each matrix coded as its own columns: codes at
    the matrix's rows (128-row blocks interleaved back for GLU), scales
    [n, matrices, 2] (sign) or [n, matrices] (trellis) flattened per column."""
    parts = _segments(w_cm, layout, seg_rows)
    if len(parts) == 1:
        return pack(w_cm, fmt, stream, codebook, **kw)
    coded = [pack(p, fmt, stream, codebook, **kw) for p in parts]
    codes = [c for c, _ in coded]
    if layout == LAYOUT_GLU_INTERLEAVED:
        # 128 rows of 2-bit codes are 32 bytes
        n, b = codes[0].shape
        g = codes[0].reshape(n, b // 32, 1, 32)
        u = codes[1].reshape(n, b // 32, 1, 32)
        codes = torch.cat([g, u], dim=2).reshape(n, 2 * b).contiguous()
    else:
        codes = torch.cat(codes, dim=1).contiguous()
    scales = torch.stack([sc for _, sc in coded], dim=1)
    return codes, scales.reshape(scales.shape[0], -1).contiguous()


def _pin(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def build_matrix(w_cm: torch.Tensor, full_fmt: int = FMT_FP16,
                 approx_fmt: int = FMT_INT4_G128, layout: int = LAYOUT_PLAIN,
                 residency: int = RES_DEVICE, stream=None,
                 codebook: Optional[torch.Tensor] = None, seg_rows: int = 0) -> Matrix:
    """A spax_matrix for a column-major fp16 device tensor [n, R].

    The full tier is w_cm itself (fp16) or its int4 code; the approx tier is
    the int4 / int2 group-128 code, the two-scale sign code or the trellis
    code of w_cm. seg_rows > 0 says w_cm stacks matrices of seg_rows rows
    (stack_rows of q, k, v); the sign and trellis codes are then fitted per
    matrix column, as they are for gate and up in the GLU layout. With
    RES_HOST_PINNED every buffer is copied to pinned host memory and the
    device copies are dropped."""
    n, R = w_cm.shape
    fs = None
    if full_fmt == FMT_FP16:
        fd = w_cm
    else:
        fd, fs = pack(w_cm, full_fmt, stream)
    ac = asc = None
    if approx_fmt in (FMT_SIGN2, FMT_TRELLIS):
        ac, asc = pack_per_matrix(w_cm, approx_fmt, layout, seg_rows, stream, codebook)
    elif approx_fmt != FMT_NONE:
        ac, asc = pack(w_cm, approx_fmt, stream, codebook)
    if residency == RES_HOST_PINNED:
        torch.cuda.synchronize()
        fd, fs, ac, asc = _pin(fd), _pin(fs), _pin(ac), _pin(asc)
    # the trellis codebook stays in device memory (the product loads it to LDS)
    cb = codebook if approx_fmt == FMT_TRELLIS else None
    return Matrix.make(R, n, full_fmt, approx_fmt, fd, fs, ac, asc, residency, layout, cb,
                       approx_seg_rows=seg_rows if layout == LAYOUT_PLAIN else 0)
