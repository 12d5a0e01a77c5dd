"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/spax.h declares, sizes workspaces, and rejects bad
arguments with the documented status codes before enqueuing any work."""
import ctypes
import os
import re

import pytest

import activation_sparse_decode_token_amd as spax

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spax.h")

# Fake, 16-byte aligned device addresses: every call below fails validation
# before it would touch them.
P = 0x10000
P2 = 0x20000


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spax_[a-z0-9_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = spax.lib()
    declared = _declared_functions()
    assert declared == sorted(spax.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert spax.version() == 200


def test_status_strings():
    for code in range(0, -9, -1):
        assert spax.status_string(code) not in ("", "unknown status")
    assert "memory" in spax.status_string(-8)
    assert spax.status_string(-99) == "unknown status"


def _matrix(rows=4096, cols=4096, ff=spax.FMT_FP16, af=spax.FMT_INT4_G128,
            res=spax.RES_DEVICE, layout=spax.LAYOUT_PLAIN):
    return spax.Matrix.make(rows, cols, ff, af, P, P if ff == spax.FMT_INT4_G128 else None,
                            P if af else None, P if af else None, res, layout)


def test_workspace_sizes():
    W = _matrix()
    ws = spax.gemv_workspace_bytes(W)
    # fixed counter region (2048 tiles x 9 counters), the layer kernel's sync
    # words (256 bytes), the sliced selection's region (16 slices of 256 +
    # 256 + 4 counts, 8 results; 256-byte padded), 64 splits of fp32 partials
    sel = (16 * (256 + 256 + 4) * 4 + 8 * 4 + 255) // 256 * 256
    head = 2048 * 9 * 4 + 256 + sel
    assert ws == head + 64 * 4096 * 4
    Wh = _matrix(res=spax.RES_HOST_PINNED)
    assert spax.gemv_workspace_bytes(Wh) >= ws + 4096 * 2 * 4096
    bad = _matrix(rows=100)
    assert spax.gemv_workspace_bytes(bad) == 0
    # staging of the sign code: rows / 4 code bytes and 2 scales per column
    Ws = _matrix(af=spax.FMT_SIGN2, res=spax.RES_HOST_PINNED)
    assert spax.gemv_workspace_bytes(Ws) == spax.gemv_workspace_bytes(Wh)
    L = spax.Layer.make([W, _matrix(), None, None], [1, 1, 0, 0], [1, 1, 0, 0])
    # the layer kernel: per group (tiles + 512 workgroups) x 512 rows of fp32
    assert spax.layer_workspace_bytes(L) == head + 2 * (8 + 512) * 512 * 4


def _gemv(W, x=P, fidx=P, kf=10, aidx=P, ka=10, y=P, ws=P2, ws_bytes=1 << 30, cp=None):
    return spax.lib().spax_tiered_gemv(ctypes.byref(W), x, fidx, kf, aidx, ka, y, ws, ws_bytes,
                                       None, cp)


def test_gemv_validation_errors():
    W = _matrix()
    assert _gemv(W, kf=-1) == -1
    assert _gemv(W, kf=3000, ka=2000) == -1
    assert _gemv(_matrix(rows=200)) == -1
    assert _gemv(_matrix(rows=spax.MAX_ROWS + 128)) == -1
    assert _gemv(_matrix(af=spax.FMT_NONE), ka=5) == -1
    assert _gemv(W, x=None) == -2
    assert _gemv(W, fidx=None) == -2
    assert _gemv(W, y=None) == -2
    assert _gemv(W, x=P + 2) == -3
    assert _gemv(_matrix(ff=spax.FMT_INT2_G128)) == -4
    assert _gemv(_matrix(af=7)) == -4
    # the trellis tier needs its codebook and an fp16 full tier
    assert _gemv(_matrix(af=spax.FMT_TRELLIS)) == -2
    Wt = spax.Matrix.make(4096, 4096, spax.FMT_FP16, spax.FMT_TRELLIS, P, None, P, P,
                          approx_codebook=P + 8)
    assert _gemv(Wt) == -3
    Wt = spax.Matrix.make(4096, 4096, spax.FMT_INT4_G128, spax.FMT_TRELLIS, P, P, P, P,
                          approx_codebook=P)
    assert _gemv(Wt) == -4
    # the sign code is an approx tier under an fp16 full tier only
    assert _gemv(_matrix(ff=spax.FMT_INT4_G128, af=spax.FMT_SIGN2)) == -4
    assert _gemv(_matrix(af=spax.FMT_SIGN2), ws_bytes=1024) == -5
    assert _gemv(W, ws_bytes=1024) == -5
    assert _gemv(_matrix(res=spax.RES_HOST_PINNED)) == -6
    # a copy context that was never set up (no stream, no events)
    assert _gemv(_matrix(res=spax.RES_HOST_PINNED), cp=ctypes.byref(spax.Copy())) == -6
    assert _gemv(_matrix(layout=spax.LAYOUT_GLU_INTERLEAVED, rows=128 * 3)) == -1
    assert spax.lib().spax_tiered_gemv(None, P, P, 1, P, 1, P, P, 1 << 30, None, None) == -2


def test_plan_validation_errors():
    f = spax.lib().spax_plan_tiers
    assert f(P, 0, 0, 0, P, P, None) == -1
    assert f(P, 65537, 1, 1, P, P, None) == -1
    assert f(P, 100, 60, 41, P, P, None) == -1
    assert f(P, 100, -1, 1, P, P, None) == -1
    assert f(None, 100, 1, 1, P, P, None) == -2
    assert f(P, 100, 1, 0, None, P, None) == -2
    assert f(P + 8, 100, 1, 1, P, P, None) == -3


def test_layer_and_helper_validation_errors():
    W = _matrix()
    gu = _matrix(rows=2 * 11008, cols=4096, layout=spax.LAYOUT_GLU_INTERLEAVED)
    dn = _matrix(rows=4096, cols=11008)
    io = spax.LayerIO.make(h=P, z=P, x=P, qkv=P, o=P, a=P, down=P, full_idx=(P,) * 4,
                           approx_idx=(P,) * 4)
    f = spax.lib().spax_layer_step
    # gate/up alone needs its output a
    L = spax.Layer.make([W, None, gu, None], [1] * 4, [1] * 4)
    io_no_a = spax.LayerIO.make(h=P, z=P, x=P, qkv=P, o=P, a=None, down=P, full_idx=(P,) * 4,
                                approx_idx=(P,) * 4)
    assert f(ctypes.byref(L), ctypes.byref(io_no_a), P2, 1 << 30, None, None) == -2
    # down needs the plain layout
    L = spax.Layer.make([None, None, None, _matrix(rows=4096, cols=11008,
                                                   layout=spax.LAYOUT_GLU_INTERLEAVED)],
                        [1] * 4, [1] * 4)
    assert f(ctypes.byref(L), ctypes.byref(io), P2, 1 << 30, None, None) == -1
    # down width must match the gate/up intermediate size
    L = spax.Layer.make([None, None, gu, _matrix(rows=4096, cols=4096)], [1] * 4, [1] * 4)
    assert f(ctypes.byref(L), ctypes.byref(io), P2, 1 << 30, None, None) == -1
    # gate/up must be GLU-interleaved
    L = spax.Layer.make([None, None, _matrix(rows=22016), dn], [1] * 4, [1] * 4)
    assert f(ctypes.byref(L), ctypes.byref(io), P2, 1 << 30, None, None) == -1
    L = spax.Layer.make([W, None, gu, dn], [1] * 4, [1] * 4)
    assert f(ctypes.byref(L), ctypes.byref(io), P2, 16, None, None) == -5
    io2 = spax.LayerIO.make(h=P, z=P, x=P, qkv=P, o=P, a=None, down=P, full_idx=(P,) * 4,
                            approx_idx=(P,) * 4)
    assert f(ctypes.byref(L), ctypes.byref(io2), P2, 1 << 30, None, None) == -2
    assert f(None, ctypes.byref(io), P2, 1 << 30, None, None) == -2
    # an unknown launch form
    L = spax.Layer.make([W, None, gu, dn], [1] * 4, [1] * 4, kernel=7)
    assert f(ctypes.byref(L), ctypes.byref(io), P2, 1 << 30, None, None) == -1
    # a workgroup cap past the partial-sum region, or negative
    for wg in (-1, 513):
        L = spax.Layer.make([W, None, gu, dn], [1] * 4, [1] * 4, workgroups=wg)
        assert f(ctypes.byref(L), ctypes.byref(io), P2, 1 << 30, None, None) == -1
    g = spax.lib().spax_pack_g128
    assert g(P, 4096, 16, spax.FMT_FP16, P, P, None) == -4
    assert g(P, 100, 16, spax.FMT_INT4_G128, P, P, None) == -1
    assert g(None, 128, 16, spax.FMT_INT2_G128, P, P, None) == -2
    import numpy as np
    tr = spax.lib().spax_pack_trellis_host
    assert tr(P, 100, 4, P, P, P, 1) == -1
    assert tr(None, 128, 4, P, P, P, 1) == -2
    assert tr(P, 128, 4, None, P, P, 1) == -2
    s2 = spax.lib().spax_pack_sign2
    assert s2(P, 100, 16, P, P, None) == -1
    assert s2(P, 128, 0, P, P, None) == -1
    assert s2(None, 128, 16, P, P, None) == -2
    assert s2(P, 128, 16, P + 4, P, None) == -3
    c = spax.lib().spax_workspace_clear
    assert c(P, 6, None) == -1
    assert c(None, 8, None) == -2
    assert c(P, 0, None) == 0
    st = spax.lib().spax_workspace_status
    assert st(None, None, 0, ctypes.byref(ctypes.c_uint32())) == -2
    assert st(P, None, 0, None) == -2
    # the copy context: a stream is required; releasing an empty one is a no-op
    ci = spax.lib().spax_copy_init
    assert ci(ctypes.byref(spax.Copy()), None) == -2
    assert ci(None, P) == -2
    assert spax.lib().spax_copy_release(ctypes.byref(spax.Copy())) == 0
    assert spax.lib().spax_copy_release(None) == -2


def test_static_layer_step_rejects_what_its_scratch_cannot_hold():
    f = spax.lib().spax_layer_step_static
    io = spax.LayerIO.make(h=P, z=P, x=P, qkv=P, o=P, a=P, down=P, full_idx=(P,) * 4,
                           approx_idx=(P,) * 4)
    assert f(None, ctypes.byref(io), None) == -2
    # a 131072-row projection's split partials alone take 32 MiB: refused
    # before any GPU call, with the reason in spax_last_error
    big = spax.Layer.make([None, _matrix(rows=131072, cols=4096), None, None], [1] * 4, [1] * 4)
    assert spax.layer_workspace_bytes(big) > 16 << 20
    assert f(ctypes.byref(big), ctypes.byref(io), None) == -5
    assert "16 MiB" in spax.last_error()
    # an empty layer
    assert f(ctypes.byref(spax.Layer.make([None] * 4, [0] * 4, [0] * 4)), ctypes.byref(io),
             None) == -1


def test_sq_error_argument_checks():
    """spax_sq_error refuses bad arguments before any GPU call."""
    f = spax.lib().spax_sq_error
    assert f(None, P, 8, P, 0, None) == -2
    assert f(P, None, 8, P, 0, None) == -2
    assert f(P, P, 8, None, 0, None) == -2
    assert f(P, P, -1, P, 0, None) == -1
    assert f(None, None, 0, None, 0, None) == -2  # the accumulator is always required
    assert f(P + 1, P, 8, P, 0, None) == -3
    assert f(P, P + 1, 8, P, 0, None) == -3
    assert f(P, P, 8, P + 4, 0, None) == -3


def test_python_wrapper_raises_with_status():
    with pytest.raises(spax.SpaxError) as ei:
        spax.plan_tiers(None, 10, 1, 1, P, P, stream=0)
    assert ei.value.status == -2
