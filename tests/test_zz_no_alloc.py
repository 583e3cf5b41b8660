"""dcn_backward_noalloc (the backward entry point that allocates nothing,
its f16/bf16 grad_x sums in the library's static scratch array) against
dcn_backward_ws with a caller workspace, through the C ABI: two calls in a
row on one GPU, the second on a smaller problem, so that the second finds
the first's sums left in the scratch and must clear what it uses."""
import ctypes

import numpy as np
import pytest

from parity_util import TOL, rel_err, say, to_dev, to_host
from sparse_deformable_sampling_amd import synth

pytestmark = pytest.mark.gpu


def _call(L, B, fn, desc, ts, outs, ws=None):
    import torch
    vp = ctypes.c_void_p
    args = [ctypes.byref(desc)] + [vp(t.data_ptr()) for t in ts] + [vp(t.data_ptr()) for t in outs]
    if ws is not None:
        args += [vp(ws.data_ptr()), ctypes.c_size_t(ws.numel() * 4)]
    args.append(vp(torch.cuda.current_stream().cuda_stream))
    return fn(*args)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    import torch
    from sparse_deformable_sampling_amd import _binding as B
    L = B.lib()
    code = {"f32": B.DCN_F32, "f16": B.DCN_F16, "bf16": B.DCN_BF16}[dtype]
    # the stage-1 shape (grad_x sums of 51.4 MB), then a smaller ragged one
    for (n, h, w, c, g), softmax, seed in (((64, 56, 56, 64, 4), False, 201), ((3, 13, 17, 32, 2), True, 202)):
        d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype=dtype, seed=seed, grad=True)
        ins = [to_dev(d[k], dtype) for k in ("x", "offset", "mask", "grad_out")]
        desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, softmax, code)
        nb = ctypes.c_size_t(0)
        assert L.dcn_backward_workspace_size(ctypes.byref(desc), ctypes.byref(nb)) == B.DCN_OK
        ws = torch.empty(((nb.value + 3) // 4,), dtype=torch.float32, device="cuda") if nb.value else None
        ref = [torch.empty_like(ins[0]), torch.empty_like(ins[1]), torch.empty_like(ins[2])]
        got = [torch.full_like(t, float("nan")) for t in ref]
        say("noalloc", dtype, (n, h, w, c, g), "softmax", softmax)
        st = _call(L, B, L.dcn_backward_ws, desc, ins, ref, ws if ws is not None else torch.empty(0, device="cuda"))
        assert st == B.DCN_OK, L.dcn_last_error()
        st = _call(L, B, L.dcn_backward_noalloc, desc, ins, got)
        assert st == B.DCN_OK, L.dcn_last_error()
        torch.cuda.synchronize()
        e = rel_err(to_host(got[0]), to_host(ref[0]))
        say("  err", "noalloc", dtype, "grad_x %.3e" % e)
        assert e <= TOL[dtype]
        # grad_offset and grad_mask take no atomics: identical bits
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
