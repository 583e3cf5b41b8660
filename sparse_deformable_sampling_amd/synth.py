"""Seeded synthetic inputs for the deformable sampling operators.

This module holds no arithmetic of the method: it draws random tensors of the
shapes and distributions of the workloads and stores them in the requested
dtype.  It is the one module that both the GPU path's callers and the CPU
oracle's callers use, so that both see identical inputs.

Generator: numpy's Philox4x32-10 counter-based bit generator (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC'11), one independent stream
per tensor, keyed by ``1000 * seed + tensor_id``.  Values are drawn in float32
and rounded to nearest-even into f16 or bf16.  bf16 tensors are returned as
their uint16 bit patterns because numpy has no bfloat16 type.
"""
from __future__ import annotations

import numpy as np

# stream ids, one per tensor
X, OFFSET, MASK, GRAD_OUT, VALUE, REF, MSDA_OFFSET, ATTN, VALID = 1, 2, 3, 4, 5, 6, 7, 8, 9
DW_WEIGHT, DW_BIAS, OM_WEIGHT, OM_BIAS, MODULE_VALUE = 10, 11, 12, 13, 14

DTYPES = ("f32", "f16", "bf16")


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=1000 * int(seed) + int(tensor_id)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in the given dtype ("f32", "f16" or "bf16")."""
    if dtype == "f32":
        return np.ascontiguousarray(a, np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(a.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError("dtype must be one of %s" % (DTYPES,))


def normal(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    r = _rng(seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        r *= np.float32(std)
    return r


def uniform(shape, lo: float, hi: float, seed: int, tensor_id: int) -> np.ndarray:
    return _rng(seed, tensor_id).uniform(lo, hi, size=shape).astype(np.float32)


def dcn_inputs(n, h, w, c, group, out_hw, taps=9, offset=("normal", 1.5), dtype="f32", seed=1,
               grad=False):
    """x ~ N(0,1) [n,h,w,c]; offsets [n,ho,wo,group,taps,2] drawn from
    ``offset`` = ("normal", std) or ("uniform", lo, hi); mask [n,ho,wo,group,taps]
    ~ N(0,1) (logits for DCNv3, raw modulation for DCNv4); optional
    grad_out ~ N(0,1) [n,ho,wo,c]."""
    ho, wo = out_hw
    out = {"x": store(normal((n, h, w, c), 1.0, seed, X), dtype)}
    oshape = (n, ho, wo, group, taps, 2)
    if offset[0] == "normal":
        off = normal(oshape, offset[1], seed, OFFSET)
    elif offset[0] == "uniform":
        off = uniform(oshape, offset[1], offset[2], seed, OFFSET)
    else:
        raise ValueError(offset)
    out["offset"] = store(off, dtype)
    out["mask"] = store(normal((n, ho, wo, group, taps), 1.0, seed, MASK), dtype)
    if grad:
        out["grad_out"] = store(normal((n, ho, wo, c), 1.0, seed, GRAD_OUT), dtype)
    return out


def frontend_inputs(n, h, w, c, group, taps=9, dtype="f16", seed=1):
    """Inputs of the DCNv4 front-end: x ~ N(0,1) [n,h,w,c]; depthwise weights
    [3,3,c] ~ N(0, 1/9) and bias [c] ~ N(0, 0.1^2); merged linear weights
    [group*taps*3, c] ~ N(0, 1/c) and bias ~ N(0, 0.1^2) (unit-scale outputs,
    like a layer at initialisation)."""
    no = group * taps * 3
    return {"x": store(normal((n, h, w, c), 1.0, seed, X), dtype),
            "dw_weight": store(normal((3, 3, c), 1.0 / 3.0, seed, DW_WEIGHT), dtype),
            "dw_bias": store(normal((c,), 0.1, seed, DW_BIAS), dtype),
            "om_weight": store(normal((no, c), float(c) ** -0.5, seed, OM_WEIGHT), dtype),
            "om_bias": store(normal((no,), 0.1, seed, OM_BIAS), dtype)}


def frontend_exact_inputs(n, h, w, c, group, taps=9, dtype="f16", seed=1):
    """Front-end inputs whose depthwise sums and offset/mask outputs are all
    exactly representable in f16 and bf16, so that no rounding happens
    between the front-end and the core op: x integers in [-2, 2], depthwise
    weights in {-1, -1/2, 0, 1/2, 1} and bias in {-1/2, 0, 1/2} (sums are
    multiples of 1/2 below 19 in magnitude); each linear row has two nonzero
    weights in {+-1/64, +-1/32} and a bias k/128 with |k| <= 32 (outputs are
    multiples of 1/128 below 3/2 in magnitude)."""
    no = group * taps * 3
    rng = _rng(seed, OM_WEIGHT)
    omw = np.zeros((no, c), np.float32)
    for j in range(no):
        cols = rng.choice(c, size=min(2, c), replace=False)
        omw[j, cols] = rng.choice([-1 / 32, -1 / 64, 1 / 64, 1 / 32], size=cols.size)
    return {"x": store(_rng(seed, X).integers(-2, 3, size=(n, h, w, c)).astype(np.float32), dtype),
            "dw_weight": store(_rng(seed, DW_WEIGHT).choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(3, 3, c))
                               .astype(np.float32), dtype),
            "dw_bias": store(_rng(seed, DW_BIAS).choice([-0.5, 0.0, 0.5], size=(c,)).astype(np.float32), dtype),
            "om_weight": store(omw, dtype),
            "om_bias": store((_rng(seed, OM_BIAS).integers(-32, 33, size=(no,)) / 128.0).astype(np.float32), dtype)}


def module_inputs(n, h, w, c, group, dtype="f16", seed=1):
    """The front-end inputs (frontend_inputs) plus the core op's value tensor
    ~ N(0,1) [n,h,w,c] (the input projection's output in a DCNv4 module)."""
    d = frontend_inputs(n, h, w, c, group, dtype=dtype, seed=seed)
    d["value"] = store(normal((n, h, w, c), 1.0, seed, MODULE_VALUE), dtype)
    return d


def msda_inputs(n, shapes, len_q, heads, head_dim, points, offset_std=2.0, dtype="f32", seed=1, ref="uniform"):
    """Value ~ N(0,1) [n,S,heads,head_dim] with S = sum H_l*W_l; per query a
    reference point; each sampling location is that point plus
    N(0, offset_std) divided by the level's (W_l, H_l); attention logits
    ~ N(0,1) [n,len_q,heads,L,points].

    ref="uniform": reference points ~ U(0,1)^2, independent per query.
    ref="cells": the encoder's queries, one per cell of the flattened maps
    (level-major, row-major, so len_q must be S), each referring to its own
    cell centre ((x + 1/2)/W_l, (y + 1/2)/H_l) (valid ratios of 1)."""
    L = len(shapes)
    S = int(sum(int(hh) * int(ww) for hh, ww in shapes))
    value = store(normal((n, S, heads, head_dim), 1.0, seed, VALUE), dtype)
    if ref == "uniform":
        ref = uniform((n, len_q, 1, 1, 1, 2), 0.0, 1.0, seed, REF)
    elif ref == "cells":
        if len_q != S:
            raise ValueError("ref='cells' needs one query per cell (len_q == %d)" % S)
        cen = []
        for hh, ww in shapes:
            yy, xx = np.meshgrid(np.arange(hh, dtype=np.float64), np.arange(ww, dtype=np.float64), indexing="ij")
            cen.append(np.stack([(xx.ravel() + 0.5) / ww, (yy.ravel() + 0.5) / hh], axis=-1))
        ref = np.broadcast_to(np.concatenate(cen).astype(np.float32).reshape(1, S, 1, 1, 1, 2), (n, S, 1, 1, 1, 2))
    else:
        raise ValueError("ref must be 'uniform' or 'cells'")
    dev = normal((n, len_q, heads, L, points, 2), offset_std, seed, MSDA_OFFSET)
    size = np.array([[ww, hh] for hh, ww in shapes], np.float32).reshape(1, 1, 1, L, 1, 2)
    loc = (ref + dev / size).astype(np.float32)
    attn = store(normal((n, len_q, heads, L, points), 1.0, seed, ATTN), dtype)
    return {"value": value, "loc": store(loc, dtype), "attn": attn}


def msda_ref_inputs(n, shapes, len_q, heads, head_dim, points, ref_dims=2, offset_std=2.0, padded=True, seed=1,
                    ref="uniform"):
    """Inputs of the reference-based MSDA read (f32):
    value ~ N(0,1) [n,S,heads,head_dim]; attn logits ~ N(0,1);
    offsets ~ N(0, offset_std) [n,q,heads,L,P,2] (pixels for point references,
    box-relative units for boxes, where +-P spans the box);
    reference [n,q,ref_dims] in valid-image coordinates: points ~ U(0,1)^2,
    boxes (x, y) ~ U(0,1)^2 with (w, h) ~ U(0.05, 0.5)^2.
    padded=True: image b keeps a fraction f_b ~ U(0.6, 1) of every level's
    width and height (at least one cell) at the top-left; the rest is
    right/bottom padding, marked in padding_mask [n,S] (1 = padded), and
    valid_ratios [n,L,2] = (valid W / W_l, valid H / H_l).  padded=False:
    ratios of 1 and no mask.
    ref="cells" (points only): the encoder's queries, one per cell of the
    flattened maps (len_q must be S), each referring to its own cell centre in
    its image's valid frame, ((x + 1/2) / (r_w W_l), (y + 1/2) / (r_h H_l))."""
    L = len(shapes)
    S = int(sum(int(hh) * int(ww) for hh, ww in shapes))
    value = normal((n, S, heads, head_dim), 1.0, seed, VALUE)
    offsets = normal((n, len_q, heads, L, points, 2), offset_std, seed, MSDA_OFFSET)
    attn = normal((n, len_q, heads, L, points), 1.0, seed, ATTN)
    if ref_dims == 2:
        reference = uniform((n, len_q, 2), 0.0, 1.0, seed, REF)
    elif ref_dims == 4:
        u = uniform((n, len_q, 4), 0.0, 1.0, seed, REF)
        reference = np.concatenate([u[..., :2], 0.05 + 0.45 * u[..., 2:]], axis=-1).astype(np.float32)
    else:
        raise ValueError("ref_dims must be 2 or 4")
    ratios = np.ones((n, L, 2), np.float32)
    mask = np.zeros((n, S), np.uint8)
    if padded:
        frac = uniform((n,), 0.6, 1.0, seed, VALID)
        start = 0
        for l, (hh, ww) in enumerate(shapes):
            for b in range(n):
                wv = max(1, int(np.ceil(frac[b] * ww)))
                hv = max(1, int(np.ceil(frac[b] * hh)))
                ratios[b, l] = (wv / ww, hv / hh)
                m = np.ones((hh, ww), np.uint8)
                m[:hv, :wv] = 0
                mask[b, start:start + hh * ww] = m.reshape(-1)
            start += hh * ww
    if ref == "cells":
        if ref_dims != 2 or len_q != S:
            raise ValueError("ref='cells' needs point references and one query per cell (len_q == %d)" % S)
        cen = []
        for l, (hh, ww) in enumerate(shapes):
            yy, xx = np.meshgrid(np.arange(hh, dtype=np.float64), np.arange(ww, dtype=np.float64), indexing="ij")
            cx = (xx.ravel()[None, :] + 0.5) / (ratios[:, l, 0:1].astype(np.float64) * ww)
            cy = (yy.ravel()[None, :] + 0.5) / (ratios[:, l, 1:2].astype(np.float64) * hh)
            cen.append(np.stack([cx, cy], axis=-1))
        reference = np.concatenate(cen, axis=1).astype(np.float32)
    elif ref != "uniform":
        raise ValueError("ref must be 'uniform' or 'cells'")
    return {"value": value, "reference": np.ascontiguousarray(reference), "offsets": offsets, "attn": attn,
            "valid_ratios": ratios if padded else None, "padding_mask": mask if padded else None}
