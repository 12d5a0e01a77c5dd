"""Python binding of libspax (three-tier activation-sparse decode on gfx950).

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI declared in include/spax.h. Device buffers are torch tensors
(or raw integer addresses); streams are torch.cuda.Stream objects or raw
hipStream_t handles. Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "SpaxError", "lib", "library_path",
    "FMT_NONE", "FMT_FP16", "FMT_INT4_G128", "FMT_INT2_G128", "FMT_SIGN2", "FMT_TRELLIS",
    "RES_DEVICE", "RES_HOST_PINNED", "LAYOUT_PLAIN", "LAYOUT_GLU_INTERLEAVED",
    "GROUP_QKV", "GROUP_O", "GROUP_GATE_UP", "GROUP_DOWN",
    "Matrix", "Layer", "LayerIO", "Copy",
    "KERNEL_AUTO", "KERNEL_SEPARATE", "KERNEL_PER_GROUP",
    "plan_tiers", "tiered_gemv", "gemv_workspace_bytes", "layer_step", "layer_step_static",
    "layer_workspace_bytes", "pack_g128", "pack_sign2", "pack_trellis_host", "pack_trellis",
    "workspace_clear", "version", "copy_init", "copy_release", "layer_schedule",
    "workspace_status",
    "status_string", "last_error", "EXPORTS",
]

FMT_NONE, FMT_FP16, FMT_INT4_G128, FMT_INT2_G128, FMT_SIGN2, FMT_TRELLIS = 0, 1, 2, 3, 4, 5
RES_DEVICE, RES_HOST_PINNED = 0, 1
LAYOUT_PLAIN, LAYOUT_GLU_INTERLEAVED = 0, 1
GROUP_QKV, GROUP_O, GROUP_GATE_UP, GROUP_DOWN = 0, 1, 2, 3
KERNEL_AUTO, KERNEL_SEPARATE, KERNEL_PER_GROUP = 0, 1, 2
COPY_CHUNKS = 4
# Fields of one spax_layer_schedule record.
SCHEDULE_FIELDS = ("workgroup", "group", "tile", "f0", "f1", "a0", "a1", "w_lo", "w_hi")
MAX_ROWS = 1 << 20

STATUS = {0: "SPAX_OK", -1: "SPAX_EINVAL", -2: "SPAX_ENULL", -3: "SPAX_EALIGN",
          -4: "SPAX_EFORMAT", -5: "SPAX_EWORKSPACE", -6: "SPAX_ESTREAM", -7: "SPAX_EHIP",
          -8: "SPAX_ENOMEM"}

# Every entry point declared in include/spax.h.
EXPORTS = (
    "spax_plan_tiers", "spax_gemv_workspace_bytes", "spax_tiered_gemv",
    "spax_layer_workspace_bytes", "spax_layer_step", "spax_pack_g128", "spax_pack_sign2",
    "spax_pack_trellis_host", "spax_pack_trellis", "spax_pack_trellis_workspace_bytes",
    "spax_workspace_clear", "spax_status_string", "spax_last_error", "spax_version",
    "spax_copy_init", "spax_copy_release", "spax_layer_schedule", "spax_workspace_status",
    "spax_layer_step_static", "spax_sq_error",
)

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspax.so")


class SpaxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({_status_text(status)})"
        if status == -7:
            msg += f": {_last_error_text()}"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspax.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: the library then binds to the HIP runtime torch has
        # loaded, so both share one runtime (devices, streams, allocations)
        import torch  # noqa: F401
        if not os.path.exists(library_path):
            raise ImportError(
                f"{library_path} is missing; build it with "
                "`python -m activation_sparse_decode_token_amd.build`")
        L = ctypes.CDLL(library_path)
        _declare(L)
        _lib = L
    return _lib


class Matrix(ctypes.Structure):
    """spax_matrix. Keeps Python references to the tensors it points to."""
    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
        ("full_fmt", ctypes.c_int32), ("approx_fmt", ctypes.c_int32),
        ("residency", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("approx_seg_rows", ctypes.c_int32),
        ("full_data", ctypes.c_void_p), ("full_scales", ctypes.c_void_p),
        ("approx_codes", ctypes.c_void_p), ("approx_scales", ctypes.c_void_p),
        ("approx_codebook", ctypes.c_void_p),
    ]

    @classmethod
    def make(cls, rows, cols, full_fmt, approx_fmt, full_data, full_scales=None,
             approx_codes=None, approx_scales=None, residency=RES_DEVICE,
             layout=LAYOUT_PLAIN, approx_codebook=None, approx_seg_rows=0) -> "Matrix":
        m = cls(rows, cols, full_fmt, approx_fmt, residency, layout, int(approx_seg_rows),
                _ptr(full_data), _ptr(full_scales), _ptr(approx_codes), _ptr(approx_scales),
                _ptr(approx_codebook))
        m._keep = (full_data, full_scales, approx_codes, approx_scales, approx_codebook)
        return m


class Layer(ctypes.Structure):
    """spax_layer: the four groups, their tier counts, the launch form
    (KERNEL_AUTO: the one-launch layer kernel where it applies) and the
    layer kernel's workgroup cap (0: one per compute unit)."""
    _fields_ = [("group", Matrix * 4), ("k_full", ctypes.c_int32 * 4),
                ("k_approx", ctypes.c_int32 * 4), ("kernel", ctypes.c_int32),
                ("workgroups", ctypes.c_int32)]

    @classmethod
    def make(cls, groups: Sequence[Optional[Matrix]], k_full: Sequence[int],
             k_approx: Sequence[int], kernel: int = KERNEL_AUTO,
             workgroups: int = 0) -> "Layer":
        L = cls()
        for g in range(4):
            if groups[g] is not None:
                L.group[g] = groups[g]
            L.k_full[g] = int(k_full[g])
            L.k_approx[g] = int(k_approx[g])
        L.kernel = int(kernel)
        L.workgroups = int(workgroups)
        L._keep = tuple(groups)
        return L


class Copy(ctypes.Structure):
    """spax_copy: the copy stream and events of host-resident products, set
    up once by copy_init and released by copy_release."""
    _fields_ = [("stream", ctypes.c_void_p), ("ready", ctypes.c_void_p),
                ("chunk", ctypes.c_void_p * COPY_CHUNKS), ("device", ctypes.c_int32)]


class LayerIO(ctypes.Structure):
    _fields_ = [
        ("h", ctypes.c_void_p), ("z", ctypes.c_void_p), ("x", ctypes.c_void_p),
        ("qkv", ctypes.c_void_p), ("o", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("u", ctypes.c_void_p), ("a", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("full_idx", ctypes.c_void_p * 4), ("approx_idx", ctypes.c_void_p * 4),
    ]

    @classmethod
    def make(cls, h=None, z=None, x=None, qkv=None, o=None, g=None, u=None, a=None,
             down=None, full_idx=(None,) * 4, approx_idx=(None,) * 4) -> "LayerIO":
        io = cls(_ptr(h), _ptr(z), _ptr(x), _ptr(qkv), _ptr(o), _ptr(g), _ptr(u), _ptr(a),
                 _ptr(down))
        for i in range(4):
            io.full_idx[i] = _ptr(full_idx[i])
            io.approx_idx[i] = _ptr(approx_idx[i])
        io._keep = (h, z, x, qkv, o, g, u, a, down, tuple(full_idx), tuple(approx_idx))
        return io


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise SpaxError(status, where)


def _status_text(status: int) -> str:
    return lib().spax_status_string(status).decode()


def _last_error_text() -> str:
    return lib().spax_last_error().decode()


def _declare(L: ctypes.CDLL) -> None:
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.spax_plan_tiers.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.spax_plan_tiers.restype = ctypes.c_int
    L.spax_gemv_workspace_bytes.argtypes = [ctypes.POINTER(Matrix)]
    L.spax_gemv_workspace_bytes.restype = sz
    L.spax_tiered_gemv.argtypes = [ctypes.POINTER(Matrix), vp, vp, i32, vp, i32, vp, vp, sz,
                                   vp, ctypes.POINTER(Copy)]
    L.spax_tiered_gemv.restype = ctypes.c_int
    L.spax_layer_workspace_bytes.argtypes = [ctypes.POINTER(Layer)]
    L.spax_layer_workspace_bytes.restype = sz
    L.spax_layer_step.argtypes = [ctypes.POINTER(Layer), ctypes.POINTER(LayerIO), vp, sz, vp,
                                  ctypes.POINTER(Copy)]
    L.spax_layer_step.restype = ctypes.c_int
    L.spax_layer_step_static.argtypes = [ctypes.POINTER(Layer), ctypes.POINTER(LayerIO), vp]
    L.spax_layer_step_static.restype = ctypes.c_int
    L.spax_sq_error.argtypes = [vp, vp, ctypes.c_int64, vp, i32, vp]
    L.spax_sq_error.restype = ctypes.c_int
    L.spax_pack_g128.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.spax_pack_g128.restype = ctypes.c_int
    L.spax_pack_sign2.argtypes = [vp, i32, i32, vp, vp, vp]
    L.spax_pack_sign2.restype = ctypes.c_int
    L.spax_pack_trellis_host.argtypes = [vp, i32, i32, vp, vp, vp, i32]
    L.spax_pack_trellis_host.restype = ctypes.c_int
    L.spax_pack_trellis.argtypes = [vp, i32, i32, vp, vp, vp, vp, sz, vp]
    L.spax_pack_trellis.restype = ctypes.c_int
    L.spax_pack_trellis_workspace_bytes.argtypes = [i32, i32]
    L.spax_pack_trellis_workspace_bytes.restype = sz
    L.spax_workspace_clear.argtypes = [vp, sz, vp]
    L.spax_workspace_clear.restype = ctypes.c_int
    L.spax_status_string.argtypes = [ctypes.c_int]
    L.spax_status_string.restype = ctypes.c_char_p
    L.spax_last_error.argtypes = []
    L.spax_last_error.restype = ctypes.c_char_p
    L.spax_version.argtypes = []
    L.spax_version.restype = ctypes.c_int
    L.spax_copy_init.argtypes = [ctypes.POINTER(Copy), vp]
    L.spax_copy_init.restype = ctypes.c_int
    L.spax_copy_release.argtypes = [ctypes.POINTER(Copy)]
    L.spax_copy_release.restype = ctypes.c_int
    i64 = ctypes.c_int64
    L.spax_layer_schedule.argtypes = [ctypes.POINTER(Layer), i32, vp, i64, ctypes.POINTER(i64)]
    L.spax_layer_schedule.restype = ctypes.c_int
    L.spax_workspace_status.argtypes = [vp, vp, i32, ctypes.POINTER(ctypes.c_uint32)]
    L.spax_workspace_status.restype = ctypes.c_int


# ---------------------------------------------------------------- entry points

def version() -> int:
    return lib().spax_version()


def status_string(status: int) -> str:
    return _status_text(status)


def last_error() -> str:
    return _last_error_text()


def plan_tiers(x, n, k_full, k_approx, full_idx, approx_idx, stream=None) -> None:
    """spax_plan_tiers: ascending full / approx index lists of x (fp16[n])."""
    _check(lib().spax_plan_tiers(_ptr(x), int(n), int(k_full), int(k_approx),
                                 _ptr(full_idx), _ptr(approx_idx), _stream(stream)),
           "spax_plan_tiers")


def gemv_workspace_bytes(W: Matrix) -> int:
    return int(lib().spax_gemv_workspace_bytes(ctypes.byref(W)))


def copy_init(copy_stream) -> Copy:
    """spax_copy_init: events for host-resident products on the current
    device, with the given copy stream (kept alive by the returned object)."""
    c = Copy()
    _check(lib().spax_copy_init(ctypes.byref(c), _stream(copy_stream)), "spax_copy_init")
    c._keep = copy_stream
    return c


def copy_release(c: Copy) -> None:
    """spax_copy_release: destroys the events of copy_init."""
    _check(lib().spax_copy_release(ctypes.byref(c)), "spax_copy_release")


def _copy_arg(copy: Optional[Copy]):
    return None if copy is None else ctypes.byref(copy)


def tiered_gemv(W: Matrix, x, full_idx, k_full, approx_idx, k_approx, y, ws, ws_bytes=None,
                stream=None, copy: Optional[Copy] = None) -> None:
    """spax_tiered_gemv: y = W[:,F] x_F + W^[:,A] x_A (fp32 accumulate, fp16 out)."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().spax_tiered_gemv(ctypes.byref(W), _ptr(x), _ptr(full_idx), int(k_full),
                                  _ptr(approx_idx), int(k_approx), _ptr(y), _ptr(ws),
                                  int(nbytes), _stream(stream), _copy_arg(copy)),
           "spax_tiered_gemv")


def layer_workspace_bytes(L: Layer) -> int:
    return int(lib().spax_layer_workspace_bytes(ctypes.byref(L)))


def layer_step(L: Layer, io: LayerIO, ws, ws_bytes=None, compute_stream=None,
               copy: Optional[Copy] = None) -> None:
    """spax_layer_step: the four ranking groups of one decoder layer."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().spax_layer_step(ctypes.byref(L), ctypes.byref(io), _ptr(ws), int(nbytes),
                                 _stream(compute_stream), _copy_arg(copy)),
           "spax_layer_step")


def layer_step_static(L: Layer, io: LayerIO, compute_stream=None) -> None:
    """spax_layer_step_static: spax_layer_step on the library's static
    scratch (no workspace, no allocation; calls on one GPU must not
    overlap)."""
    _check(lib().spax_layer_step_static(ctypes.byref(L), ctypes.byref(io),
                                        _stream(compute_stream)),
           "spax_layer_step_static")


def layer_schedule(L: Layer, workgroups: int = 0):
    """spax_layer_schedule: the layer kernel's work pieces as an int32 array
    of shape [count, 9] (fields SCHEDULE_FIELDS)."""
    import numpy as np
    count = ctypes.c_int64(0)
    _check(lib().spax_layer_schedule(ctypes.byref(L), int(workgroups), None, 0,
                                     ctypes.byref(count)), "spax_layer_schedule")
    out = np.zeros((count.value, 9), dtype=np.int32)
    if count.value:
        _check(lib().spax_layer_schedule(ctypes.byref(L), int(workgroups), out.ctypes.data,
                                         count.value, ctypes.byref(count)),
               "spax_layer_schedule")
    return out


def workspace_status(ws, stream=None, reset: bool = False) -> int:
    """spax_workspace_status: the layer kernel's sticky status bits in ws."""
    v = ctypes.c_uint32(0)
    _check(lib().spax_workspace_status(_ptr(ws), _stream(stream), int(bool(reset)),
                                       ctypes.byref(v)), "spax_workspace_status")
    return int(v.value)


def sq_error(y, ref, n, acc, accumulate: bool = False, stream=None) -> None:
    """spax_sq_error: sum_i (y_i - ref_i)^2 in fp64 into (or onto) acc[0]."""
    _check(lib().spax_sq_error(_ptr(y), _ptr(ref), int(n), _ptr(acc), int(bool(accumulate)),
                               _stream(stream)),
           "spax_sq_error")


def pack_g128(w, rows, cols, fmt, codes, scales, stream=None) -> None:
    """spax_pack_g128: int4 / int2 group-128 codes and fp16 scales of w."""
    _check(lib().spax_pack_g128(_ptr(w), int(rows), int(cols), int(fmt), _ptr(codes),
                                _ptr(scales), _stream(stream)),
           "spax_pack_g128")


def pack_sign2(w, rows, cols, codes, scales, stream=None) -> None:
    """spax_pack_sign2: two-scale 2-bit sign codes and fp16 (s0, s1) of w."""
    _check(lib().spax_pack_sign2(_ptr(w), int(rows), int(cols), _ptr(codes), _ptr(scales),
                                 _stream(stream)),
           "spax_pack_sign2")


def pack_trellis_host(w, rows, cols, codebook, codes, scales, threads=None) -> None:
    """spax_pack_trellis_host: trellis codes and fp16 scales of w (host numpy
    arrays: w fp16 [cols, rows], codebook fp16 [65536], codes uint8
    [cols, rows/4], scales fp16 [cols])."""
    import numpy as np
    for a, dt in ((w, np.float16), (codebook, np.float16), (codes, np.uint8),
                  (scales, np.float16)):
        if not (isinstance(a, np.ndarray) and a.dtype == dt and a.flags.c_contiguous):
            raise TypeError("pack_trellis_host takes C-contiguous numpy arrays")
    n = threads if threads else max(1, min(16, os.cpu_count() or 1))
    _check(lib().spax_pack_trellis_host(w.ctypes.data, int(rows), int(cols), codebook.ctypes.data,
                                        codes.ctypes.data, scales.ctypes.data, int(n)),
           "spax_pack_trellis_host")


def pack_trellis(w, rows, cols, codebook, codes, scales, ws, ws_bytes=None,
                 stream=None) -> None:
    """spax_pack_trellis: the trellis encoding on the GPU (device tensors)."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().spax_pack_trellis(_ptr(w), int(rows), int(cols), _ptr(codebook), _ptr(codes),
                                   _ptr(scales), _ptr(ws), int(nbytes), _stream(stream)),
           "spax_pack_trellis")


def pack_trellis_workspace_bytes(rows, batch) -> int:
    return int(lib().spax_pack_trellis_workspace_bytes(int(rows), int(batch)))


def workspace_clear(ws, nbytes=None, stream=None) -> None:
    n = ws.numel() * ws.element_size() if nbytes is None else nbytes
    _check(lib().spax_workspace_clear(_ptr(ws), int(n), _stream(stream)), "spax_workspace_clear")
