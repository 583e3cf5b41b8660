"""CPU checks of the device code as compiled for gfx950 (no GPU needed): the
hot-path kernels keep every value in registers.  A kernel near its register
budget (the 1024-thread forward variants are held to 128 VGPRs) can tip into
scratch spills after a small source change, which costs several times its run
time without changing any result, so the parity tests cannot see it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_deformable_sampling_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HOT_SOURCES = ["dcn_forward_ring.hip", "dcn_backward_win.hip", "msda_forward.hip", "msda_backward.hip",
               "dcn_frontend.hip"]


def kernel_resources(src, tmp_path):
    from sparse_deformable_sampling_amd import build
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.check_call([HIPCC] + flags + ["-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                                             "-o", out, os.path.join(CSRC, src)],
                          stderr=subprocess.DEVNULL)
    text = open(out).read()
    res = {}
    for block in re.findall(r"\.name:\s+(\S+)(.*?)(?=\n\s+- \.|\Z)", text, flags=re.S):
        name, body = block
        m = re.search(r"\.vgpr_spill_count:\s+(\d+)", body)
        if m:
            res[name] = int(m.group(1))
    return res


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", HOT_SOURCES)
def test_hot_kernels_do_not_spill(src, tmp_path):
    res = kernel_resources(src, tmp_path)
    assert res, "no kernels found in %s" % src
    spilled = {k: v for k, v in res.items() if v}
    assert not spilled, spilled
