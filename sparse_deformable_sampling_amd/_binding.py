"""ctypes binding of libdcn's C ABI (include/dcn.h).

Argument marshalling only: shapes are checked, pointers and the current HIP
stream are passed, and every step of the computation runs in the HIP
kernels.  If libdcn.so is missing or cannot be loaded the calls raise; there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LIBDCN_PATH names another build of the same library (the sanitized host
# build the CPU tests load); the default is the in-tree libdcn.so.
LIB_PATH = os.environ.get("LIBDCN_PATH") or os.path.join(HERE, "libdcn.so")

DCN_OK, DCN_ERR_INVALID, DCN_ERR_UNSUPPORTED, DCN_ERR_HIP = 0, 1, 2, 3
DCN_F32, DCN_F16, DCN_BF16 = 0, 1, 2


class DcnDesc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("n", "h", "w", "c", "group", "kernel_h", "kernel_w", "stride_h", "stride_w",
                 "pad_h", "pad_w", "dil_h", "dil_w")] + [
        ("offset_scale", ctypes.c_float), ("softmax", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class MsdaDesc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("n", "len_q", "heads", "head_dim", "levels", "points", "softmax", "dtype")]


EXPORTS = ("dcn_output_size", "dcn_forward", "dcn_backward", "dcn_backward_workspace_size", "dcn_backward_ws",
           "dcn_backward_noalloc", "dcn_offset_mask",
           "msda_forward", "msda_forward_ref", "msda_backward", "msda_backward_workspace_size", "msda_backward_ws",
           "dcn_status_str", "dcn_last_error")

_lib = None


def lib():
    """Load libdcn.so (building it first if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) and "LIBDCN_PATH" not in os.environ:
        from . import build as _build
        _build.build()
    _lib = load(LIB_PATH)
    return _lib


COUNT_LIB_PATH = os.path.join(HERE, "libdcn_count.so")
_count_lib = None


def count_lib():
    """The write-counting debug build, libdcn_count.so (include/dcn_debug.h):
    the entry points of libdcn.so plus dcn_debug_count_writes.  Built by
    build.build(); loaded only by tests."""
    global _count_lib
    if _count_lib is None:
        if not os.path.exists(COUNT_LIB_PATH):
            raise FileNotFoundError("%s is not built (sparse_deformable_sampling_amd.build.build())" % COUNT_LIB_PATH)
        L = load(COUNT_LIB_PATH)
        L.dcn_debug_count_writes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        L.dcn_debug_count_writes.restype = ctypes.c_int
        _count_lib = L
    return _count_lib


def load(path):
    """Open a build of libdcn at path and declare its entry points' argument types."""
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.dcn_output_size.argtypes = [ctypes.POINTER(DcnDesc), ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32)]
    L.dcn_output_size.restype = ctypes.c_int
    L.dcn_forward.argtypes = [ctypes.POINTER(DcnDesc), vp, vp, vp, vp, vp]
    L.dcn_forward.restype = ctypes.c_int
    L.dcn_backward.argtypes = [ctypes.POINTER(DcnDesc), vp, vp, vp, vp, vp, vp, vp, vp]
    L.dcn_backward.restype = ctypes.c_int
    L.dcn_backward_workspace_size.argtypes = [ctypes.POINTER(DcnDesc), ctypes.POINTER(ctypes.c_size_t)]
    L.dcn_backward_workspace_size.restype = ctypes.c_int
    L.dcn_backward_ws.argtypes = [ctypes.POINTER(DcnDesc), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dcn_backward_ws.restype = ctypes.c_int
    L.dcn_backward_noalloc.argtypes = [ctypes.POINTER(DcnDesc), vp, vp, vp, vp, vp, vp, vp, vp]
    L.dcn_backward_noalloc.restype = ctypes.c_int
    L.msda_forward.argtypes = [ctypes.POINTER(MsdaDesc), ctypes.POINTER(ctypes.c_int32), vp, vp, vp, vp, vp]
    L.msda_forward.restype = ctypes.c_int
    L.dcn_offset_mask.argtypes = [ctypes.POINTER(DcnDesc), vp, vp, vp, vp, vp, vp, vp, vp]
    L.dcn_offset_mask.restype = ctypes.c_int
    L.msda_forward_ref.argtypes = [ctypes.POINTER(MsdaDesc), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, vp, vp, vp,
                                   vp, vp, vp, vp, vp]
    L.msda_forward_ref.restype = ctypes.c_int
    L.msda_backward.argtypes = [ctypes.POINTER(MsdaDesc), ctypes.POINTER(ctypes.c_int32), vp, vp, vp, vp, vp, vp, vp,
                                vp]
    L.msda_backward.restype = ctypes.c_int
    L.msda_backward_workspace_size.argtypes = [ctypes.POINTER(MsdaDesc), ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_size_t)]
    L.msda_backward_workspace_size.restype = ctypes.c_int
    L.msda_backward_ws.argtypes = [ctypes.POINTER(MsdaDesc), ctypes.POINTER(ctypes.c_int32), vp, vp, vp, vp, vp, vp,
                                   vp, vp, ctypes.c_size_t, vp]
    L.msda_backward_ws.restype = ctypes.c_int
    L.dcn_status_str.argtypes = [ctypes.c_int]
    L.dcn_status_str.restype = ctypes.c_char_p
    L.dcn_last_error.argtypes = []
    L.dcn_last_error.restype = ctypes.c_char_p
    return L


class DcnError(RuntimeError):
    def __init__(self, status: int):
        L = lib()
        self.status = status
        super().__init__("%s: %s" % (L.dcn_status_str(status).decode(), L.dcn_last_error().decode()))


def check(status: int) -> None:
    if status != DCN_OK:
        raise DcnError(status)


def _pair(v):
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def make_desc(n, h, w, c, group, kernel=3, stride=1, pad=1, dil=1, offset_scale=1.0, softmax=False,
              dtype=DCN_F32) -> DcnDesc:
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dil)
    return DcnDesc(n, h, w, c, group, kh, kw, sh, sw, ph, pw, dh, dw, float(offset_scale), int(bool(softmax)),
                   int(dtype))


def output_size(desc: DcnDesc):
    ho, wo = ctypes.c_int32(), ctypes.c_int32()
    check(lib().dcn_output_size(ctypes.byref(desc), ctypes.byref(ho), ctypes.byref(wo)))
    return ho.value, wo.value
