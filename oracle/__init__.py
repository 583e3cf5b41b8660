"""CPU oracle for the deformable sampling operators -- TEST INFRASTRUCTURE ONLY.

Plain, slow, single-threaded and double precision.  Only ``tests/``, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product library (``sparse_deformable_sampling_amd``)
never imports it, and the two share no code.

The sampling arithmetic lives in ``dcn_oracle.c`` (compiled with gcc into
``oracle/_build/liboracle.so``); this module converts the stored input values
to float64 exactly and marshals the arrays.  Two groups of functions here are
numpy float64 written out from their definitions: the MSDA reference-to-
location formula (``msda_locations``) and the DCNv4 front-end (the depthwise
3x3 sum and the merged linear, ``depthwise3x3``, ``dcnv4_offset_mask``).
Every function states the passage of the pages it follows:

* "InternImage: Deformable Convolutions at Scale", Ch.2-4 (bilinear read,
  DCNv3 operator and softmax, groups);
* "DCNv4: Unbounded Weights", "Why Is Sampling Just 9 Points Still Slow?" and
  "1. Remove Softmax" (the per-group sum, unnormalised modulation, the merged
  offset/modulation linear after a depthwise 3x3);
* "Deformable DETR: Learn Where to Read", "A learned location can fall between
  cells" and "Mix samples with a per-head budget" (MSDA sampling and joint
  softmax); "A reference links resolutions without equating their pixels"
  (locations from references and valid ratios).

Conventions no number in the pages fixes (tap order, offset pair order,
offset_scale, the front-end's output order) are parity unpinned; every other
function is pinned in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcn_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                  "-shared-libsan"]


def build_sanitized(path: str, cc: str = "/opt/rocm/llvm/bin/clang") -> str:
    """Compile the C oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    into ``path`` (clang, so that it shares one sanitizer runtime with the
    sanitized host build of libdcn).  The process that loads it must preload
    that runtime; ORACLE_LIB_PATH=path makes this module load it."""
    subprocess.check_call([cc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"] +
                          SANITIZE_FLAGS + ["-o", path, _SRC, "-lm"])
    return path


class _Dcn(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in
                ("n", "h", "w", "c", "group", "kernel_h", "kernel_w", "stride_h", "stride_w",
                 "pad_h", "pad_w", "dil_h", "dil_w")] + [
        ("offset_scale", ctypes.c_double), ("softmax", ctypes.c_int)]


class _Msda(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in
                ("n", "len_q", "heads", "head_dim", "levels", "points", "softmax")]


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB_PATH names another build of dcn_oracle.c (the sanitized
        # one); the default is the gcc build above.
        path = os.environ.get("ORACLE_LIB_PATH") or build(force=False)
        lib = ctypes.CDLL(path)
        pd = ctypes.POINTER(ctypes.c_double)
        lib.oracle_dcn_out_size.argtypes = [ctypes.POINTER(_Dcn), ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(ctypes.c_int)]
        for name in ("oracle_dcn_forward", "oracle_dcn_forward_tent"):
            getattr(lib, name).argtypes = [ctypes.POINTER(_Dcn), pd, pd, pd, pd]
        lib.oracle_dcn_backward.argtypes = [ctypes.POINTER(_Dcn), pd, pd, pd, pd, pd, pd, pd]
        for name in ("oracle_msda_forward", "oracle_msda_forward_tent"):
            getattr(lib, name).argtypes = [ctypes.POINTER(_Msda), ctypes.POINTER(ctypes.c_int),
                                           pd, pd, pd, pd]
        lib.oracle_msda_backward.argtypes = [ctypes.POINTER(_Msda), ctypes.POINTER(ctypes.c_int),
                                             pd, pd, pd, pd, pd, pd, pd]
        _lib = lib
    return _lib


def to_f64(a: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Exact float64 copy of stored values.  bf16 arrives as its uint16 bit
    pattern (numpy has no bfloat16): the bits are the top half of an f32."""
    if dtype == "bf16" or (dtype is None and a.dtype == np.uint16):
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dcn_struct(n, h, w, c, group, kernel, stride, pad, dil, offset_scale, softmax):
    kh, kw = kernel
    return _Dcn(n, h, w, c, group, kh, kw, stride[0], stride[1], pad[0], pad[1],
                dil[0], dil[1], float(offset_scale), int(softmax))


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def dcn_out_size(h, w, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dil=(1, 1)):
    p = _dcn_struct(1, h, w, 1, 1, _pair(kernel), _pair(stride), _pair(pad), _pair(dil), 1.0, 0)
    ho, wo = ctypes.c_int(), ctypes.c_int()
    _load().oracle_dcn_out_size(ctypes.byref(p), ctypes.byref(ho), ctypes.byref(wo))
    return ho.value, wo.value


def dcn_forward(x, offset, mask, group, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dil=(1, 1),
                offset_scale=1.0, softmax=False, dtype=None, tent=False):
    """out[n,ho,wo,c] of the DCN core op, float64.  x: [n,h,w,c];
    offset: [n,ho,wo,group,K,2] holding (dx, dy); mask: [n,ho,wo,group,K]."""
    x64, o64, m64 = to_f64(x, dtype), to_f64(offset, dtype), to_f64(mask, dtype)
    n, h, w, c = x64.shape
    kernel, stride, pad, dil = _pair(kernel), _pair(stride), _pair(pad), _pair(dil)
    p = _dcn_struct(n, h, w, c, group, kernel, stride, pad, dil, offset_scale, softmax)
    ho, wo = dcn_out_size(h, w, kernel, stride, pad, dil)
    K = kernel[0] * kernel[1]
    assert o64.size == n * ho * wo * group * K * 2 and m64.size == n * ho * wo * group * K
    out = np.zeros((n, ho, wo, c), np.float64)
    fn = _load().oracle_dcn_forward_tent if tent else _load().oracle_dcn_forward
    rc = fn(ctypes.byref(p), _ptr(x64), _ptr(np.ascontiguousarray(o64)), _ptr(np.ascontiguousarray(m64)),
            _ptr(out))
    assert rc == 0
    return out


def dcn_backward(x, offset, mask, grad_out, group, kernel=(3, 3), stride=(1, 1), pad=(1, 1),
                 dil=(1, 1), offset_scale=1.0, softmax=False, dtype=None):
    """(grad_x, grad_offset, grad_mask) in float64; grad_mask is with respect
    to the values passed in mask (the logits when softmax is set)."""
    x64, o64, m64 = to_f64(x, dtype), to_f64(offset, dtype), to_f64(mask, dtype)
    g64 = to_f64(grad_out, dtype)
    n, h, w, c = x64.shape
    kernel, stride, pad, dil = _pair(kernel), _pair(stride), _pair(pad), _pair(dil)
    p = _dcn_struct(n, h, w, c, group, kernel, stride, pad, dil, offset_scale, softmax)
    gx = np.zeros_like(x64)
    go = np.zeros(o64.shape, np.float64)
    gm = np.zeros(m64.shape, np.float64)
    rc = _load().oracle_dcn_backward(ctypes.byref(p), _ptr(x64), _ptr(np.ascontiguousarray(o64)),
                                     _ptr(np.ascontiguousarray(m64)), _ptr(np.ascontiguousarray(g64)),
                                     _ptr(gx), _ptr(go), _ptr(gm))
    assert rc == 0
    return gx, go, gm


def depthwise3x3(x, weight, bias, dtype=None):
    """Depthwise 3x3 convolution, stride 1, zero padding 1, float64: the first
    half of the DCNv4 offset subnetwork, a separable convolution ("DCNv4:
    Unbounded Weights", "1. Remove Softmax").  x: [n,h,w,c]; weight:
    [3][3][c] (row, column, channel); bias: [c].  Written as the direct sum
    out[y,x,c] = bias[c] + sum_{i,j} weight[i,j,c] * x[y+i-1, x+j-1, c]."""
    x64, w64, b64 = to_f64(x, dtype), to_f64(weight, dtype), to_f64(bias, dtype)
    n, h, w, c = x64.shape
    xp = np.zeros((n, h + 2, w + 2, c))
    xp[:, 1:-1, 1:-1] = x64
    out = np.broadcast_to(b64, (n, h, w, c)).copy()
    for i in range(3):
        for j in range(3):
            out += w64[i, j] * xp[:, i:i + h, j:j + w]
    return out


def dcnv4_offset_mask(x, dw_weight, dw_bias, om_weight, om_bias, group, taps=9, dtype=None):
    """Offsets [n,h,w,group,taps,2] and mask [n,h,w,group,taps] (float64) of
    the DCNv4 front-end: the depthwise 3x3 convolution, then ONE linear layer
    that predicts offsets and modulation together ("DCNv4...", "1. Remove
    Softmax": merged offset and weight linears, no softmax, no LayerNorm or
    GELU between the two halves).  om_weight: [group*taps*3][c] (output x
    input, as a linear layer stores it), om_bias: [group*taps*3]; output channels 0 .. group*taps*2-1 are
    the offsets in [group][taps][2] order, the rest the mask in [group][taps]
    order."""
    d = depthwise3x3(x, dw_weight, dw_bias, dtype)
    n, h, w, c = d.shape
    om = d.reshape(-1, c) @ to_f64(om_weight, dtype).T + to_f64(om_bias, dtype)
    no = group * taps * 2
    offset = om[:, :no].reshape(n, h, w, group, taps, 2)
    mask = om[:, no:].reshape(n, h, w, group, taps)
    return offset, mask


def msda_forward(value, shapes, loc, attn, softmax=True, dtype=None, tent=False):
    """out[n,q,heads,head_dim] of multi-scale deformable attention, float64.
    value: [n,S,heads,head_dim]; shapes: [(H_l, W_l)]; loc: [n,q,heads,L,P,2]
    normalised (u, v); attn: [n,q,heads,L,P] (logits when softmax is set)."""
    v64, l64, a64 = to_f64(value, dtype), to_f64(loc, dtype), to_f64(attn, dtype)
    n, S, M, Dh = v64.shape
    _, Q, M2, L, P, two = l64.shape
    assert M2 == M and two == 2 and len(shapes) == L
    sh = np.ascontiguousarray(np.asarray(shapes, np.int32).reshape(L, 2))
    assert int((sh[:, 0].astype(np.int64) * sh[:, 1]).sum()) == S
    p = _Msda(n, Q, M, Dh, L, P, int(softmax))
    out = np.zeros((n, Q, M, Dh), np.float64)
    fn = _load().oracle_msda_forward_tent if tent else _load().oracle_msda_forward
    rc = fn(ctypes.byref(p), sh.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _ptr(v64),
            _ptr(np.ascontiguousarray(l64)), _ptr(np.ascontiguousarray(a64)), _ptr(out))
    assert rc == 0
    return out


def msda_locations(reference, offsets, shapes, valid_ratios=None):
    """Sampling locations [n,q,heads,L,P,2] (float64) formed from references
    and offsets.

    "Deformable DETR: Learn Where to Read", "A reference links resolutions
    without equating their pixels" and "Math and tensor shapes": a point
    reference p (valid-image coordinates) maps into level l's padded frame as
    p * r_l, and the offset is divided by the level's (W_l, H_l); for a box
    reference (x, y, w, h) the offset term is instead (offset / P) * (w, h) *
    r_l / 2, with P the points per level ("A learned location can fall between
    cells", on box references).  r_l = (valid W / W_l, valid H / H_l) per
    image; no clamping.
    reference: [n,q,2] or [n,q,4]; offsets: [n,q,heads,L,P,2];
    valid_ratios: [n,L,2] or None (ratios of 1)."""
    ref = to_f64(reference)
    off = to_f64(offsets)
    n, Q, M, L, P, two = off.shape
    assert two == 2 and ref.shape[:2] == (n, Q) and ref.shape[2] in (2, 4) and len(shapes) == L
    ratios = np.ones((n, L, 2)) if valid_ratios is None else to_f64(valid_ratios)
    loc = np.zeros(off.shape, np.float64)
    for b in range(n):
        for q in range(Q):
            for l in range(L):
                size = (shapes[l][1], shapes[l][0])          # (W_l, H_l)
                for axis in range(2):
                    centre = ref[b, q, axis] * ratios[b, l, axis]
                    if ref.shape[2] == 4:
                        shift = off[b, q, :, l, :, axis] / P * ref[b, q, axis + 2] * ratios[b, l, axis] * 0.5
                    else:
                        shift = off[b, q, :, l, :, axis] / size[axis]
                    loc[b, q, :, l, :, axis] = centre + shift
    return loc


def msda_forward_ref(value, shapes, reference, offsets, attn, valid_ratios=None, padding_mask=None, softmax=True):
    """msda_forward at the locations of msda_locations, after zeroing the
    value cells marked in padding_mask [n,S] (the attention module zeroes
    projected values at masked positions: "Deformable DETR...", "A reference
    links resolutions without equating their pixels")."""
    v64 = to_f64(value).copy()
    if padding_mask is not None:
        v64[np.asarray(padding_mask).astype(bool)] = 0.0
    loc = msda_locations(reference, offsets, shapes, valid_ratios)
    return msda_forward(v64, shapes, loc, attn, softmax=softmax)


def msda_backward(value, shapes, loc, attn, grad_out, softmax=True, dtype=None):
    """(grad_value, grad_loc, grad_attn) of msda_forward in float64;
    grad_attn is with respect to the values passed in attn (the logits when
    softmax is set)."""
    v64, l64, a64 = to_f64(value, dtype), to_f64(loc, dtype), to_f64(attn, dtype)
    g64 = to_f64(grad_out, dtype)
    n, S, M, Dh = v64.shape
    _, Q, M2, L, P, two = l64.shape
    assert M2 == M and two == 2 and len(shapes) == L and g64.shape == (n, Q, M, Dh)
    sh = np.ascontiguousarray(np.asarray(shapes, np.int32).reshape(L, 2))
    assert int((sh[:, 0].astype(np.int64) * sh[:, 1]).sum()) == S
    p = _Msda(n, Q, M, Dh, L, P, int(softmax))
    gv = np.zeros_like(v64)
    gl = np.zeros(l64.shape, np.float64)
    ga = np.zeros(a64.shape, np.float64)
    rc = _load().oracle_msda_backward(ctypes.byref(p), sh.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _ptr(v64),
                                      _ptr(np.ascontiguousarray(l64)), _ptr(np.ascontiguousarray(a64)),
                                      _ptr(np.ascontiguousarray(g64)), _ptr(gv), _ptr(gl), _ptr(ga))
    assert rc == 0
    return gv, gl, ga
