"""One writer per output element: the forward kernels are atomic-free, so every
element of dcn_forward's output (and of msda_forward / msda_forward_ref's, on
their vector paths, and of dcn_offset_mask's two outputs) must be stored
exactly once, and no store may land outside the outputs.  The debug build libdcn_count.so counts every output store per
element (include/dcn_debug.h); these tests run the ops through it, in the
launch configurations the library picks at the workloads' full sizes and on
the fallback kernels, and check every count and that the outputs equal the
product library's bit for bit."""
import ctypes

import numpy as np
import pytest

import oracle
from parity_util import say, to_dev
from sparse_deformable_sampling_amd import _binding as B, synth

pytestmark = pytest.mark.gpu

CODE = {"f32": B.DCN_F32, "f16": B.DCN_F16, "bf16": B.DCN_BF16}


@pytest.fixture(scope="module")
def sds():
    import torch
    import sparse_deformable_sampling_amd as m
    assert torch.cuda.is_available()
    B.count_lib()
    return m


def counted(monkeypatch, out, dtype, launch):
    """Run launch() with every library call routed to libdcn_count.so and the
    writes into `out` counted; returns counts[0..n] as numpy."""
    import torch
    L = B.count_lib()
    n = out.numel()
    counts = torch.zeros(n + 1, dtype=torch.int32, device=out.device)
    torch.cuda.synchronize()
    B.check(L.dcn_debug_count_writes(ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(out.data_ptr()), n,
                                     CODE[dtype]))
    try:
        with monkeypatch.context() as mp:
            mp.setattr(B, "lib", B.count_lib)
            launch()
        torch.cuda.synchronize()
    finally:
        B.check(L.dcn_debug_count_writes(None, None, 0, CODE[dtype]))
    return counts.cpu().numpy()


def check_counts(name, counts):
    n = counts.size - 1
    bad = np.flatnonzero(counts[:n] != 1)
    say("  counts", name, "elements %d, not written once %d, stray stores %d" % (n, bad.size, counts[n]))
    assert bad.size == 0, (name, bad[:8], counts[bad[:8]])
    assert counts[n] == 0, (name, "stores outside the output", int(counts[n]))


DCN_CASES = [
    # name, (n, h, w, c, g), dtype, softmax, geometry
    ("stage1-dcnv4", (64, 56, 56, 64, 4), "f16", False, {}),
    ("stage1-dcnv3", (64, 56, 56, 64, 4), "f32", True, {}),
    ("stage1-dcnv4", (64, 56, 56, 64, 4), "bf16", False, {}),
    ("stage2", (64, 28, 28, 128, 8), "bf16", False, {}),
    ("stage3", (64, 14, 14, 320, 20), "f16", False, {}),
    ("table10", (16, 56, 56, 128, 4), "f32", False, {}),
    ("wide-rows", (1, 6, 1200, 64, 4), "f16", False, {}),
    ("kernel5", (2, 12, 10, 32, 2), "f32", False, {"kernel": 5, "pad": 2}),
    ("odd-group", (2, 9, 11, 12, 2), "f32", True, {}),
    ("stride2-dil2", (2, 17, 19, 32, 2), "f16", False, {"stride": 2, "pad": 2, "dil": 2}),
]


@pytest.mark.parametrize("name,shape,dtype,softmax,geom", DCN_CASES)
def test_dcn_forward_one_writer_per_output(sds, monkeypatch, name, shape, dtype, softmax, geom):
    import torch
    n, h, w, c, g = shape
    ho, wo = oracle.dcn_out_size(h, w, geom.get("kernel", 3), geom.get("stride", 1), geom.get("pad", 1),
                                 geom.get("dil", 1))
    K = geom.get("kernel", 3) ** 2
    d = synth.dcn_inputs(n, h, w, c, g, (ho, wo), taps=K, dtype=dtype, seed=5)
    x, off, mask = (to_dev(d[k], dtype) for k in ("x", "offset", "mask"))
    say("write-count", name, dtype, shape, geom)
    out = torch.full((n, ho, wo, c), float("nan"), dtype=x.dtype, device="cuda")
    counts = counted(monkeypatch, out, dtype,
                     lambda: sds.dcn_forward(x, off, mask, group=g, softmax=softmax, out=out, **geom))
    check_counts(name, counts)
    ref = sds.dcn_forward(x, off, mask, group=g, softmax=softmax, **geom)
    assert torch.equal(out.view(torch.int16 if dtype != "f32" else torch.int32),
                       ref.view(torch.int16 if dtype != "f32" else torch.int32))


MSDA_SHAPES = [(100, 134), (50, 67), (25, 34), (13, 17)]


@pytest.mark.parametrize("ref", ["loc", "points", "boxes"])
def test_msda_forward_one_writer_per_output(sds, monkeypatch, ref):
    import torch
    n, heads, dh, pts = 2, 8, 32, 4
    S = sum(a * b for a, b in MSDA_SHAPES)
    say("write-count msda", ref, (n, S, heads, dh, pts))
    out = torch.full((n, S, heads, dh), float("nan"), dtype=torch.float32, device="cuda")
    if ref == "loc":
        d = synth.msda_inputs(n, MSDA_SHAPES, S, heads, dh, pts, seed=5, ref="cells")
        v, loc, attn = (to_dev(d[k], "f32") for k in ("value", "loc", "attn"))
        counts = counted(monkeypatch, out, "f32", lambda: sds.msda_forward(v, MSDA_SHAPES, loc, attn, out=out))
        again = sds.msda_forward(v, MSDA_SHAPES, loc, attn)
    else:
        d = synth.msda_ref_inputs(n, MSDA_SHAPES, S, heads, dh, pts, ref_dims=2 if ref == "points" else 4, seed=5)
        t = {k: to_dev(d[k], "f32") for k in ("value", "reference", "offsets", "attn", "valid_ratios")}
        args = (t["value"], MSDA_SHAPES, t["reference"], t["offsets"], t["attn"])
        kw = {"valid_ratios": t["valid_ratios"], "padding_mask": torch.from_numpy(d["padding_mask"]).cuda()}
        counts = counted(monkeypatch, out, "f32", lambda: sds.msda_forward_ref(*args, out=out, **kw))
        again = sds.msda_forward_ref(*args, **kw)
    check_counts("msda-" + ref, counts)
    assert torch.equal(out.view(torch.int32), again.view(torch.int32))


FRONTEND_CASES = [
    # name, (n, h, w, c, g), dtype: the wave kernel (C=64/128), its one-workgroup-per-CU launch, the
    # tile kernel (C=320) and a ragged map whose pixel count is not a whole number of blocks
    ("stage1", (64, 56, 56, 64, 4), "f16"),
    ("table10", (64, 56, 56, 128, 4), "bf16"),
    ("one-block", (48, 28, 28, 128, 8), "f16"),
    ("stage3", (64, 14, 14, 320, 20), "f16"),
    ("stage3", (64, 14, 14, 320, 20), "bf16"),
    ("ragged", (3, 13, 11, 96, 2), "f16"),
]


@pytest.mark.parametrize("name,shape,dtype", FRONTEND_CASES)
def test_frontend_one_writer_per_output(sds, name, shape, dtype):
    """dcn_offset_mask writes two outputs: with the offsets registered, every
    offset element is stored once and the stores outside them are exactly the
    mask's elements; then the same with the mask registered.  Called through
    the debug build's C ABI on preallocated outputs."""
    import torch
    n, h, w, c, g = shape
    d = synth.frontend_inputs(n, h, w, c, g, dtype=dtype, seed=7)
    t = {k: to_dev(v, dtype) for k, v in d.items()}
    say("write-count front-end", name, dtype, shape)
    ref_off, ref_mask = sds.dcnv4_offset_mask(t["x"], t["dw_weight"], t["dw_bias"], t["om_weight"], t["om_bias"],
                                              group=g)
    L = B.count_lib()
    desc = B.make_desc(n, h, w, c, g, kernel=3, stride=1, pad=1, dil=1, dtype=CODE[dtype])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda a: ctypes.c_void_p(a.data_ptr())
    for which in ("offset", "mask"):
        off = torch.full_like(ref_off, float("nan"))
        mask = torch.full_like(ref_mask, float("nan"))
        reg, other = (off, mask) if which == "offset" else (mask, off)
        counts = torch.zeros(reg.numel() + 1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        B.check(L.dcn_debug_count_writes(ptr(counts), ptr(reg), reg.numel(), CODE[dtype]))
        try:
            B.check(L.dcn_offset_mask(ctypes.byref(desc), ptr(t["x"]), ptr(t["dw_weight"]), ptr(t["dw_bias"]),
                                      ptr(t["om_weight"]), ptr(t["om_bias"]), ptr(off), ptr(mask), stream))
            torch.cuda.synchronize()
        finally:
            B.check(L.dcn_debug_count_writes(None, None, 0, CODE[dtype]))
        cnt = counts.cpu().numpy()
        m = cnt.size - 1
        bad = np.flatnonzero(cnt[:m] != 1)
        say("  counts", name, which, "elements %d, not written once %d, other output's stores %d (expected %d)"
            % (m, bad.size, cnt[m], other.numel()))
        assert bad.size == 0, (name, which, bad[:8], cnt[bad[:8]])
        assert cnt[m] == other.numel(), (name, which, int(cnt[m]), other.numel())
        assert torch.equal(off.view(torch.int16), ref_off.view(torch.int16))
        assert torch.equal(mask.view(torch.int16), ref_mask.view(torch.int16))
