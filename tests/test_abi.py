"""CPU tests of the C-ABI library: it loads, exports every symbol that
include/dcn.h declares, computes output sizes like the oracle, and rejects
invalid arguments before touching the GPU.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import oracle
from sparse_deformable_sampling_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dcn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:dcn_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    # exported as C symbols (no C++ mangling)
    raw = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_debug_build_exports_the_write_counter():
    """libdcn_count.so (the write-counting debug build) exports what
    include/dcn.h and include/dcn_debug.h declare; libdcn.so does not carry
    the debug entry point.  A bad dtype is rejected before any HIP call."""
    if not os.path.exists(B.COUNT_LIB_PATH):
        pytest.skip("libdcn_count.so not built")
    debug_h = open(os.path.join(os.path.dirname(HEADER), "dcn_debug.h")).read()
    debug_h = re.sub(r"/\*.*?\*/", "", debug_h, flags=re.S)
    debug = re.findall(r"^\s*dcn_status\s+(\w+)\s*\(", debug_h, flags=re.M)
    assert debug == ["dcn_debug_count_writes"]
    L = B.count_lib()
    for name in declared_functions() + debug:
        assert hasattr(L, name), name
    assert not hasattr(ctypes.CDLL(B.LIB_PATH), "dcn_debug_count_writes")
    assert L.dcn_debug_count_writes(None, None, 0, 7) == B.DCN_ERR_INVALID
    assert L.dcn_debug_count_writes(ctypes.c_void_p(64), None, 16, B.DCN_F32) == B.DCN_ERR_INVALID


def test_struct_layouts_match_header():
    # the header's structs are all 4-byte fields
    assert ctypes.sizeof(B.DcnDesc) == 16 * 4
    assert ctypes.sizeof(B.MsdaDesc) == 8 * 4


def test_status_strings():
    L = B.lib()
    assert L.dcn_status_str(0) == b"DCN_OK"
    assert L.dcn_status_str(1) == b"DCN_ERR_INVALID"
    assert L.dcn_status_str(2) == b"DCN_ERR_UNSUPPORTED"
    assert L.dcn_status_str(3) == b"DCN_ERR_HIP"


@pytest.mark.parametrize("h,w,kernel,stride,pad,dil", [
    (56, 56, 3, 1, 1, 1), (8, 8, 3, 1, 1, 1), (7, 9, (3, 2), (2, 1), (1, 2), (1, 2)),
    (28, 28, 3, 2, 1, 1), (5, 6, (1, 1), 1, 0, 1), (13, 17, (2, 3), (1, 2), (2, 0), (3, 1)),
    (1, 1, 3, 1, 1, 1), (3, 100, (3, 5), (1, 4), (0, 2), (1, 3))])
def test_output_size_matches_oracle(h, w, kernel, stride, pad, dil):
    d = B.make_desc(2, h, w, 8, 2, kernel, stride, pad, dil)
    assert B.output_size(d) == oracle.dcn_out_size(h, w, kernel, stride, pad, dil)


def _call_forward(desc, ptrs=(0x1000, 0x2000, 0x3000, 0x4000)):
    L = B.lib()
    p = [ctypes.c_void_p(v) if v else None for v in ptrs]
    return L.dcn_forward(ctypes.byref(desc) if desc is not None else None, *p, None)


BAD_DESCS = [
    dict(c=10, group=4),          # c % group
    dict(n=0), dict(h=0), dict(w=-1), dict(c=0), dict(group=0),
    dict(kernel=(0, 3)), dict(stride=(1, 0)), dict(dil=(0, 1)), dict(pad=(-1, 0)),
    dict(h=2, w=2, kernel=5, pad=0),          # kernel larger than the padded input
    dict(softmax=2), dict(dtype=7),
    dict(offset_scale=float("inf")), dict(offset_scale=float("nan")),
    dict(n=4096, h=1024, w=1024, c=1),        # 2^32 elements
    dict(h=1 << 24, w=1, c=1, group=1),       # side >= 2^24
]


@pytest.mark.parametrize("bad", BAD_DESCS)
def test_forward_rejects_invalid_descriptors(bad):
    kw = dict(n=1, h=8, w=8, c=16, group=2, kernel=3, stride=1, pad=1, dil=1)
    kw.update(bad)
    dtype = kw.pop("dtype", B.DCN_F32)
    softmax = kw.pop("softmax", 0)
    scale = kw.pop("offset_scale", 1.0)
    desc = B.make_desc(**kw, offset_scale=scale, dtype=dtype)
    desc.softmax = softmax
    st = _call_forward(desc)
    assert st == B.DCN_ERR_INVALID, B.lib().dcn_last_error()
    assert B.lib().dcn_last_error() != b""


def test_forward_rejects_null_pointers_and_desc():
    desc = B.make_desc(1, 8, 8, 16, 2)
    assert _call_forward(None) == B.DCN_ERR_INVALID
    for i in range(4):
        ptrs = [0x1000, 0x2000, 0x3000, 0x4000]
        ptrs[i] = 0
        assert _call_forward(desc, ptrs) == B.DCN_ERR_INVALID


def test_forward_rejects_misaligned_pointers():
    desc = B.make_desc(1, 8, 8, 16, 2)
    assert _call_forward(desc, (0x1002, 0x2000, 0x3000, 0x4000)) == B.DCN_ERR_UNSUPPORTED
    desc.dtype = B.DCN_F16
    assert _call_forward(desc, (0x1001, 0x2000, 0x3000, 0x4000)) == B.DCN_ERR_UNSUPPORTED


def test_backward_workspace_and_nulls():
    """f16/bf16 backward with grad_x sums in a caller-provided fp32 workspace:
    its size is 4*n*h*w*c (0 for f32); a missing, short or misaligned one is
    rejected before any launch."""
    L = B.lib()
    vp = ctypes.c_void_p
    nbytes = ctypes.c_size_t(123)
    for dt, want in ((B.DCN_F16, 4 * 8 * 8 * 16), (B.DCN_BF16, 4 * 8 * 8 * 16), (B.DCN_F32, 0)):
        desc = B.make_desc(1, 8, 8, 16, 2, dtype=dt)
        assert L.dcn_backward_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)) == B.DCN_OK
        assert nbytes.value == want
    assert L.dcn_backward_workspace_size(ctypes.byref(desc), None) == B.DCN_ERR_INVALID
    desc = B.make_desc(1, 8, 8, 16, 2, dtype=B.DCN_F16)
    ins = (vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000))
    st = L.dcn_backward(ctypes.byref(desc), *ins, vp(0x5000), None, None, None)
    assert st == B.DCN_ERR_INVALID and b"workspace" in L.dcn_last_error()
    st = L.dcn_backward_ws(ctypes.byref(desc), *ins, vp(0x5000), None, None, vp(0x6000), 4095, None)
    assert st == B.DCN_ERR_INVALID
    st = L.dcn_backward_ws(ctypes.byref(desc), *ins, vp(0x5000), None, None, vp(0x6002), 4096, None)
    assert st == B.DCN_ERR_UNSUPPORTED
    desc = B.make_desc(1, 8, 8, 16, 2)
    st = L.dcn_backward(ctypes.byref(desc), vp(0x1000), vp(0x2000), None, vp(0x4000), vp(0x5000), None, None, None)
    assert st == B.DCN_ERR_INVALID
    # nothing requested: a valid no-op, no launch
    st = L.dcn_backward(ctypes.byref(desc), *ins, None, None, None, None)
    assert st == B.DCN_OK
    desc = B.make_desc(1, 8, 8, 16, 2, dtype=B.DCN_BF16)
    st = L.dcn_backward_ws(ctypes.byref(desc), *ins, None, None, None, None, 0, None)
    assert st == B.DCN_OK


def test_backward_noalloc_rejects_beyond_its_scratch():
    """dcn_backward_noalloc keeps f16/bf16 grad_x sums in a 64 MiB static
    array: 16 Mi elements fit, one more is refused before anything is
    enqueued (and before the array's address is looked up); invalid
    arguments are refused as by dcn_backward_ws."""
    L = B.lib()
    vp = ctypes.c_void_p
    ins = (vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000))
    desc = B.make_desc(1, 4097, 4096, 1, 1, dtype=B.DCN_F16)   # 16 Mi + 4096 elements
    st = L.dcn_backward_noalloc(ctypes.byref(desc), *ins, vp(0x5000), None, None, None)
    assert st == B.DCN_ERR_INVALID and b"scratch" in L.dcn_last_error()
    desc = B.make_desc(1, 8, 8, 16, 2, dtype=B.DCN_BF16)
    st = L.dcn_backward_noalloc(ctypes.byref(desc), vp(0x1000), None, vp(0x3000), vp(0x4000), vp(0x5000), None,
                                None, None)
    assert st == B.DCN_ERR_INVALID
    st = L.dcn_backward_noalloc(ctypes.byref(desc), *ins, vp(0x5001), None, None, None)
    assert st == B.DCN_ERR_UNSUPPORTED
    # nothing requested: a valid no-op, no launch and no scratch
    assert L.dcn_backward_noalloc(ctypes.byref(desc), *ins, None, None, None, None) == B.DCN_OK


def test_msda_validation():
    L = B.lib()
    vp = ctypes.c_void_p
    shapes = (ctypes.c_int32 * 4)(4, 5, 2, 3)
    ok = dict(n=1, len_q=3, heads=2, head_dim=8, levels=2, points=2, softmax=1, dtype=B.DCN_F32)

    def call(shp=shapes, ptrs=(0x1000, 0x2000, 0x3000, 0x4000), **over):
        d = dict(ok)
        d.update(over)
        desc = B.MsdaDesc(**d)
        return L.msda_forward(ctypes.byref(desc), shp, *[vp(p) if p else None for p in ptrs], None)

    assert call(levels=0) == B.DCN_ERR_INVALID
    assert call(points=0) == B.DCN_ERR_INVALID
    assert call(softmax=3) == B.DCN_ERR_INVALID
    assert call(dtype=9) == B.DCN_ERR_INVALID
    assert call(shp=None) == B.DCN_ERR_INVALID
    assert call(shp=(ctypes.c_int32 * 4)(4, 0, 2, 3)) == B.DCN_ERR_INVALID
    assert call(ptrs=(0x1000, 0, 0x3000, 0x4000)) == B.DCN_ERR_INVALID
    assert call(levels=17, shp=(ctypes.c_int32 * 34)(*([2] * 34))) == B.DCN_ERR_UNSUPPORTED
    assert call(dtype=B.DCN_F16) == B.DCN_ERR_UNSUPPORTED
    assert call(ptrs=(0x1002, 0x2000, 0x3000, 0x4000)) == B.DCN_ERR_UNSUPPORTED
    assert call(n=1 << 20, len_q=1 << 12) == B.DCN_ERR_INVALID


def test_msda_backward_validation():
    L = B.lib()
    vp = ctypes.c_void_p
    shapes = (ctypes.c_int32 * 4)(4, 5, 2, 3)
    ok = dict(n=1, len_q=3, heads=2, head_dim=8, levels=2, points=2, softmax=1, dtype=B.DCN_F32)
    inputs = (0x1000, 0x2000, 0x3000, 0x4000)   # value, loc, attn, grad_out

    def call(shp=shapes, ins=inputs, grads=(0x5000, 0x6000, 0x7000), **over):
        d = dict(ok)
        d.update(over)
        desc = B.MsdaDesc(**d)
        args = [vp(p) if p else None for p in tuple(ins) + tuple(grads)]
        return L.msda_backward(ctypes.byref(desc), shp, *args, None)

    assert call(levels=0) == B.DCN_ERR_INVALID
    assert call(head_dim=0) == B.DCN_ERR_INVALID
    assert call(softmax=2) == B.DCN_ERR_INVALID
    assert call(dtype=7) == B.DCN_ERR_INVALID
    assert call(shp=None) == B.DCN_ERR_INVALID
    assert call(shp=(ctypes.c_int32 * 4)(4, 5, -1, 3)) == B.DCN_ERR_INVALID
    assert call(ins=(0x1000, 0x2000, 0x3000, 0)) == B.DCN_ERR_INVALID      # grad_out is required
    assert call(ins=(0, 0x2000, 0x3000, 0x4000)) == B.DCN_ERR_INVALID
    assert call(dtype=B.DCN_BF16) == B.DCN_ERR_UNSUPPORTED
    assert call(grads=(0x5002, 0x6000, 0x7000)) == B.DCN_ERR_UNSUPPORTED  # misaligned grad_value
    assert call(grads=(0x5000, 0x6001, 0x7000)) == B.DCN_ERR_UNSUPPORTED
    assert call(levels=17, shp=(ctypes.c_int32 * 34)(*([2] * 34))) == B.DCN_ERR_UNSUPPORTED
    assert call(n=1 << 20, len_q=1 << 12) == B.DCN_ERR_INVALID
    # nothing requested: nothing is enqueued
    assert call(grads=(0, 0, 0)) == B.DCN_OK


def test_msda_backward_workspace_size_and_validation():
    """Workspace of the per-cell gather: 4 bytes per bucket of a (H_l+1) x
    (W_l+1) grid per level, image and head (plus one per pair), 20 bytes per
    sample, each part rounded up to 256 bytes; 0 where the shape has no gather
    path.  msda_backward_ws refuses a missing, short or misaligned one."""
    L = B.lib()
    vp = ctypes.c_void_p

    def size(shp, **over):
        d = dict(n=2, len_q=7, heads=3, head_dim=8, levels=len(shp) // 2, points=2, softmax=1, dtype=B.DCN_F32)
        d.update(over)
        out = ctypes.c_size_t(123)
        st = L.msda_backward_workspace_size(ctypes.byref(B.MsdaDesc(**d)), (ctypes.c_int32 * len(shp))(*shp),
                                            ctypes.byref(out))
        return st, out.value

    def up(x):
        return (x + 255) // 256 * 256

    buckets = (4 + 1) * (5 + 1) + (2 + 1) * (3 + 1)
    samples = 2 * 7 * 3 * 2 * 2
    assert size((4, 5, 2, 3)) == (B.DCN_OK, up(2 * 3 * (buckets + 1) * 4) + up(samples * 4) + samples * 16)
    enc = (100, 134, 50, 67, 25, 34, 13, 17)
    st, nb = size(enc, n=8, len_q=17821, heads=8, head_dim=32, points=4)
    assert st == B.DCN_OK and 360e6 < nb < 380e6
    assert size((4, 5, 2, 3), head_dim=36) == (B.DCN_OK, 0)     # not a power of two
    assert size((4, 5, 2, 3), head_dim=2) == (B.DCN_OK, 0)      # under 4 channels
    assert size((4, 5, 2, 3), points=3) == (B.DCN_OK, 0)        # 6 samples per head
    assert size((4, 5, 2, 3), dtype=B.DCN_F16) == (B.DCN_OK, 0)
    assert size((4, 5, 2, 3), levels=0)[0] == B.DCN_ERR_INVALID
    assert L.msda_backward_workspace_size(ctypes.byref(B.MsdaDesc(1, 3, 2, 8, 2, 2, 1, B.DCN_F32)),
                                          (ctypes.c_int32 * 4)(4, 5, 2, 3), None) == B.DCN_ERR_INVALID

    shapes = (ctypes.c_int32 * 4)(4, 5, 2, 3)
    desc = B.MsdaDesc(1, 3, 2, 8, 2, 2, 1, B.DCN_F32)
    need = ctypes.c_size_t(0)
    assert L.msda_backward_workspace_size(ctypes.byref(desc), shapes, ctypes.byref(need)) == B.DCN_OK
    ins = [vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000)]

    def call(grads=(0x5000, 0x6000, 0x7000), ws=0x100000, nbytes=None):
        g = [vp(p) if p else None for p in grads]
        return L.msda_backward_ws(ctypes.byref(desc), shapes, *ins, *g, vp(ws) if ws else None,
                                  need.value if nbytes is None else nbytes, None)

    assert call(ws=0) == B.DCN_ERR_INVALID                           # grad_value needs the workspace
    assert call(nbytes=need.value - 1) == B.DCN_ERR_INVALID
    assert call(ws=0x100010) == B.DCN_ERR_UNSUPPORTED                # not 256-byte aligned
    assert call(grads=(0, 0, 0), ws=0) == B.DCN_OK                   # nothing requested, nothing enqueued


def test_torch_wrappers_refuse_cpu_tensors():
    import torch
    import sparse_deformable_sampling_amd as sds
    x = torch.zeros(1, 4, 4, 4)
    off = torch.zeros(1, 4, 4, 1, 9, 2)
    mask = torch.zeros(1, 4, 4, 1, 9)
    with pytest.raises(RuntimeError, match="GPU"):
        sds.dcn_forward(x, off, mask, group=1)


def test_msda_forward_ref_validation():
    """ref_dims must be 2 or 4, the tensors must be given, f32 only; all
    checked before any launch."""
    L = B.lib()
    vp = ctypes.c_void_p
    shapes = (ctypes.c_int32 * 4)(4, 5, 2, 3)
    desc = B.MsdaDesc(1, 6, 2, 8, 2, 2, 1, B.DCN_F32)
    good = (vp(0x1000), vp(0x2000), None, vp(0x3000), vp(0x4000), None, vp(0x5000))

    def call(ref_dims, args):
        return L.msda_forward_ref(ctypes.byref(desc), shapes, ref_dims, *args[:6], args[6], None)

    assert call(3, good) == B.DCN_ERR_INVALID
    assert call(2, (vp(0x1000), None) + good[2:]) == B.DCN_ERR_INVALID
    assert call(4, good[:3] + (None,) + good[4:]) == B.DCN_ERR_INVALID
    assert call(2, good[:6] + (None,)) == B.DCN_ERR_INVALID
    assert call(2, (vp(0x1000), vp(0x2002)) + good[2:]) == B.DCN_ERR_UNSUPPORTED
    assert call(2, good[:2] + (vp(0x2001),) + good[3:]) == B.DCN_ERR_UNSUPPORTED
    desc.dtype = B.DCN_F16
    assert call(2, good) == B.DCN_ERR_UNSUPPORTED


def test_offset_mask_validation():
    """The DCNv4 front-end takes f16/bf16, c % 8 == 0, an output the size of
    the input and all seven tensors (16-byte aligned but for om_bias); each violation is refused before any launch."""
    L = B.lib()
    vp = ctypes.c_void_p
    good = [vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), vp(0x7000)]

    def call(desc, args=good):
        return L.dcn_offset_mask(ctypes.byref(desc), *args, None)

    assert call(B.make_desc(1, 8, 8, 16, 2)) == B.DCN_ERR_UNSUPPORTED           # f32
    assert call(B.make_desc(1, 8, 8, 12, 2, dtype=B.DCN_F16)) == B.DCN_ERR_UNSUPPORTED   # c % 8
    assert call(B.make_desc(1, 8, 8, 16, 2, stride=2, dtype=B.DCN_F16)) == B.DCN_ERR_UNSUPPORTED
    assert call(B.make_desc(1, 8, 8, 16, 2, pad=0, dtype=B.DCN_F16)) == B.DCN_ERR_UNSUPPORTED
    desc = B.make_desc(1, 8, 8, 16, 2, dtype=B.DCN_BF16)
    for i in range(7):
        args = list(good)
        args[i] = None
        assert call(desc, args) == B.DCN_ERR_INVALID, i
    for i, p in ((0, 0x1008), (1, 0x2008), (2, 0x3004), (3, 0x4008), (4, 0x5001), (5, 0x6008), (6, 0x7004)):
        args = list(good)
        args[i] = vp(p)
        assert call(desc, args) == B.DCN_ERR_UNSUPPORTED, i
    assert L.dcn_offset_mask(None, *good, None) == B.DCN_ERR_INVALID
