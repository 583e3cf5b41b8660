"""libdcn: deformable sampling-and-aggregation on AMD Instinct MI355X (gfx950).

Python face of the C ABI in ``include/dcn.h``.  The functions below carry the
same names as the C entry points and only marshal arguments: torch supplies
device memory and the current HIP stream, every step of the computation runs
in libdcn's HIP kernels.  There is no CPU path: without the built library (or
without a GPU) the calls raise.

* ``dcn_forward``  -- DCNv3 (``softmax=True``) / DCNv4 (``softmax=False``) core op
  (f32, f16, bf16; fp32 accumulation).
* ``dcn_backward`` -- its gradients (f32, f16, bf16; an f16/bf16 grad_x is
  summed in an fp32 workspace this wrapper allocates with torch).
* ``dcnv4_offset_mask`` -- the DCNv4 front-end: depthwise 3x3, then the merged
  offset/modulation linear (f16, bf16).
* ``msda_forward`` / ``msda_forward_ref`` -- multi-scale deformable attention
  sampling core, from given locations or from references (f32).
* ``msda_backward`` -- its gradients (f32).
* ``dcn_output_size`` -- output spatial size for a geometry.

Layouts: x [n,h,w,c] (NHWC); offset [n,ho,wo,group,K,2] holding (dx, dy);
mask [n,ho,wo,group,K]; out [n,ho,wo,c]; value [n,S,heads,head_dim];
loc [n,q,heads,L,P,2] holding normalised (u, v); attn [n,q,heads,L,P].
"""
from __future__ import annotations

import ctypes

from . import _binding as _b

__all__ = ["dcn_output_size", "dcn_forward", "dcn_backward", "dcnv4_offset_mask", "msda_forward", "msda_forward_ref",
           "msda_backward", "DcnError"]

DcnError = _b.DcnError


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    codes = {torch.float32: _b.DCN_F32, torch.float16: _b.DCN_F16, torch.bfloat16: _b.DCN_BF16}
    if t.dtype not in codes:
        raise TypeError("unsupported dtype %s (float32, float16 or bfloat16)" % t.dtype)
    return codes[t.dtype]


def _check_tensors(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise RuntimeError("libdcn runs on the GPU only; got a tensor on %s" % dev)
    for t in ts:
        if t.device != dev:
            raise RuntimeError("all tensors must be on one device")
        if not t.is_contiguous():
            raise RuntimeError("all tensors must be contiguous")
        if t.dtype != ts[0].dtype:
            raise RuntimeError("all tensors must share one dtype")
    return dev


def _stream(dev):
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def dcn_output_size(h, w, kernel=3, stride=1, pad=1, dil=1):
    """(ho, wo) of the DCN op for an h x w input."""
    return _b.output_size(_b.make_desc(1, h, w, 1, 1, kernel, stride, pad, dil))


def _desc_for(x, offset, mask, group, kernel, stride, pad, dil, offset_scale, softmax):
    if x.dim() != 4:
        raise ValueError("x must be [n, h, w, c]")
    n, h, w, c = x.shape
    desc = _b.make_desc(n, h, w, c, group, kernel, stride, pad, dil, offset_scale, softmax, _dtype_code(x))
    ho, wo = _b.output_size(desc)
    K = desc.kernel_h * desc.kernel_w
    if tuple(offset.shape) != (n, ho, wo, group, K, 2):
        raise ValueError("offset must be %s, got %s" % ((n, ho, wo, group, K, 2), tuple(offset.shape)))
    if tuple(mask.shape) != (n, ho, wo, group, K):
        raise ValueError("mask must be %s, got %s" % ((n, ho, wo, group, K), tuple(mask.shape)))
    return desc, (n, ho, wo, c)


def dcn_forward(x, offset, mask, group, kernel=3, stride=1, pad=1, dil=1, offset_scale=1.0, softmax=False,
                out=None):
    """DCN core op on the GPU.  ``softmax=True``: DCNv3 (mask holds logits,
    softmax over the K taps); ``softmax=False``: DCNv4 (mask used as given)."""
    dev = _check_tensors(x, offset, mask)
    desc, oshape = _desc_for(x, offset, mask, group, kernel, stride, pad, dil, offset_scale, softmax)
    if out is None:
        out = _torch().empty(oshape, dtype=x.dtype, device=dev)
    else:
        _check_tensors(x, out)
        if tuple(out.shape) != oshape:
            raise ValueError("out must be %s" % (oshape,))
    _b.check(_b.lib().dcn_forward(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask), _ptr(out), _stream(dev)))
    return out


def dcn_backward(x, offset, mask, grad_out, group, kernel=3, stride=1, pad=1, dil=1, offset_scale=1.0,
                 softmax=False, need_x=True, need_offset=True, need_mask=True):
    """(grad_x, grad_offset, grad_mask) of dcn_forward; an output not needed is None.
    f16/bf16 tensors: grad_x is summed in an fp32 workspace allocated here."""
    dev = _check_tensors(x, offset, mask, grad_out)
    desc, oshape = _desc_for(x, offset, mask, group, kernel, stride, pad, dil, offset_scale, softmax)
    if tuple(grad_out.shape) != oshape:
        raise ValueError("grad_out must be %s" % (oshape,))
    torch = _torch()
    gx = torch.empty_like(x) if need_x else None
    go = torch.empty_like(offset) if need_offset else None
    gm = torch.empty_like(mask) if need_mask else None
    nbytes = ctypes.c_size_t(0)
    _b.check(_b.lib().dcn_backward_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)))
    ws = torch.empty(((nbytes.value + 3) // 4,), dtype=torch.float32, device=dev) if (need_x and nbytes.value) \
        else None
    _b.check(_b.lib().dcn_backward_ws(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask), _ptr(grad_out),
                                      _ptr(gx), _ptr(go), _ptr(gm), _ptr(ws), nbytes.value if ws is not None else 0,
                                      _stream(dev)))
    return gx, go, gm


def dcnv4_offset_mask(x, dw_weight, dw_bias, om_weight, om_bias, group, kernel=3, pad=None, dil=1):
    """DCNv4 front-end on the GPU: (offset [n,h,w,group,K,2], mask
    [n,h,w,group,K]) from x [n,h,w,c] through the depthwise 3x3 convolution
    (dw_weight [3,3,c], dw_bias [c]) and the merged linear (om_weight
    [group*K*3, c], om_bias [group*K*3]).  f16 or bf16."""
    dev = _check_tensors(x, dw_weight, dw_bias, om_weight, om_bias)
    kh, kw = (kernel, kernel) if isinstance(kernel, int) else kernel
    dh, dw = (dil, dil) if isinstance(dil, int) else dil
    if pad is None:
        pad = ((kh - 1) * dh // 2, (kw - 1) * dw // 2)
    n, h, w, c = x.shape
    K = kh * kw
    if tuple(dw_weight.shape) != (3, 3, c) or tuple(dw_bias.shape) != (c,) or \
            tuple(om_weight.shape) != (group * K * 3, c) or tuple(om_bias.shape) != (group * K * 3,):
        raise ValueError("dw_weight [3,3,c], dw_bias [c], om_weight [group*K*3, c], om_bias [group*K*3] expected")
    torch = _torch()
    offset = torch.empty((n, h, w, group, K, 2), dtype=x.dtype, device=dev)
    mask = torch.empty((n, h, w, group, K), dtype=x.dtype, device=dev)
    desc, _ = _desc_for(x, offset, mask, group, (kh, kw), 1, pad, (dh, dw), 1.0, False)
    _b.check(_b.lib().dcn_offset_mask(ctypes.byref(desc), _ptr(x), _ptr(dw_weight), _ptr(dw_bias), _ptr(om_weight),
                                      _ptr(om_bias), _ptr(offset), _ptr(mask), _stream(dev)))
    return offset, mask


def msda_forward(value, spatial_shapes, loc, attn, softmax=True, out=None):
    """Multi-scale deformable attention sampling core on the GPU.
    spatial_shapes: sequence of (H_l, W_l)."""
    dev = _check_tensors(value, loc, attn)
    n, S, M, Dh = value.shape
    if loc.dim() != 6 or loc.shape[-1] != 2:
        raise ValueError("loc must be [n, q, heads, L, P, 2]")
    _, Q, M2, L, P, _ = loc.shape
    if loc.shape[0] != n or M2 != M or tuple(attn.shape) != (n, Q, M, L, P) or len(spatial_shapes) != L:
        raise ValueError("inconsistent value/loc/attn/spatial_shapes")
    shapes = (ctypes.c_int32 * (2 * L))(*[int(v) for hw in spatial_shapes for v in hw])
    if sum(int(h) * int(w) for h, w in spatial_shapes) != S:
        raise ValueError("sum of H_l*W_l must equal value.shape[1]")
    desc = _b.MsdaDesc(n, Q, M, Dh, L, P, int(bool(softmax)), _dtype_code(value))
    if out is None:
        out = _torch().empty((n, Q, M, Dh), dtype=value.dtype, device=dev)
    _b.check(_b.lib().msda_forward(ctypes.byref(desc), shapes, _ptr(value), _ptr(loc), _ptr(attn), _ptr(out),
                                   _stream(dev)))
    return out


def msda_forward_ref(value, spatial_shapes, reference, offsets, attn, valid_ratios=None, padding_mask=None,
                     softmax=True, out=None):
    """msda_forward with locations formed on the GPU from reference points
    ([n, q, 2]) or boxes ([n, q, 4]), valid ratios ([n, L, 2] or None) and
    offsets ([n, q, heads, L, P, 2]); padding_mask ([n, S] bool/uint8 or None)
    marks value cells that read zero."""
    dev = _check_tensors(value, reference, offsets, attn, *([] if valid_ratios is None else [valid_ratios]))
    n, S, M, Dh = value.shape
    if offsets.dim() != 6 or offsets.shape[-1] != 2:
        raise ValueError("offsets must be [n, q, heads, L, P, 2]")
    _, Q, M2, L, P, _ = offsets.shape
    if offsets.shape[0] != n or M2 != M or tuple(attn.shape) != (n, Q, M, L, P) or len(spatial_shapes) != L:
        raise ValueError("inconsistent value/offsets/attn/spatial_shapes")
    if reference.dim() != 3 or tuple(reference.shape[:2]) != (n, Q) or reference.shape[2] not in (2, 4):
        raise ValueError("reference must be [n, q, 2] or [n, q, 4]")
    if valid_ratios is not None and tuple(valid_ratios.shape) != (n, L, 2):
        raise ValueError("valid_ratios must be [n, L, 2]")
    if padding_mask is not None:
        torch = _torch()
        if tuple(padding_mask.shape) != (n, S) or padding_mask.device != value.device:
            raise ValueError("padding_mask must be [n, S] on value's device")
        padding_mask = padding_mask.to(torch.uint8).contiguous()
    shapes = (ctypes.c_int32 * (2 * L))(*[int(v) for hw in spatial_shapes for v in hw])
    if sum(int(h) * int(w) for h, w in spatial_shapes) != S:
        raise ValueError("sum of H_l*W_l must equal value.shape[1]")
    desc = _b.MsdaDesc(n, Q, M, Dh, L, P, int(bool(softmax)), _dtype_code(value))
    if out is None:
        out = _torch().empty((n, Q, M, Dh), dtype=value.dtype, device=dev)
    _b.check(_b.lib().msda_forward_ref(ctypes.byref(desc), shapes, int(reference.shape[2]), _ptr(value),
                                       _ptr(reference), _ptr(valid_ratios), _ptr(offsets), _ptr(attn),
                                       _ptr(padding_mask), _ptr(out), _stream(dev)))
    return out


def msda_backward(value, spatial_shapes, loc, attn, grad_out, softmax=True, need_value=True, need_loc=True,
                  need_attn=True, gather=True):
    """Gradients (grad_value, grad_loc, grad_attn) of msda_forward; a
    gradient that is not needed comes back as None and is not computed.
    gather=True: grad_value is gathered per value cell through a device
    workspace allocated here (no atomics into grad_value); gather=False: it is
    scattered with fp32 atomics."""
    dev = _check_tensors(value, loc, attn, grad_out)
    n, S, M, Dh = value.shape
    if loc.dim() != 6 or loc.shape[-1] != 2:
        raise ValueError("loc must be [n, q, heads, L, P, 2]")
    _, Q, M2, L, P, _ = loc.shape
    if (loc.shape[0] != n or M2 != M or tuple(attn.shape) != (n, Q, M, L, P) or len(spatial_shapes) != L
            or tuple(grad_out.shape) != (n, Q, M, Dh)):
        raise ValueError("inconsistent value/loc/attn/grad_out/spatial_shapes")
    shapes = (ctypes.c_int32 * (2 * L))(*[int(v) for hw in spatial_shapes for v in hw])
    if sum(int(h) * int(w) for h, w in spatial_shapes) != S:
        raise ValueError("sum of H_l*W_l must equal value.shape[1]")
    desc = _b.MsdaDesc(n, Q, M, Dh, L, P, int(bool(softmax)), _dtype_code(value))
    torch = _torch()
    gv = torch.empty_like(value) if need_value else None
    gl = torch.empty_like(loc) if need_loc else None
    ga = torch.empty_like(attn) if need_attn else None
    if not gather:
        _b.check(_b.lib().msda_backward(ctypes.byref(desc), shapes, _ptr(value), _ptr(loc), _ptr(attn),
                                        _ptr(grad_out), _ptr(gv), _ptr(gl), _ptr(ga), _stream(dev)))
        return gv, gl, ga
    nbytes = ctypes.c_size_t(0)
    _b.check(_b.lib().msda_backward_workspace_size(ctypes.byref(desc), shapes, ctypes.byref(nbytes)))
    ws = torch.empty((nbytes.value,), dtype=torch.uint8, device=dev) if (need_value and nbytes.value) else None
    _b.check(_b.lib().msda_backward_ws(ctypes.byref(desc), shapes, _ptr(value), _ptr(loc), _ptr(attn),
                                       _ptr(grad_out), _ptr(gv), _ptr(gl), _ptr(ga), _ptr(ws),
                                       nbytes.value if ws is not None else 0, _stream(dev)))
    return gv, gl, ga
