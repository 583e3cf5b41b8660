"""Helpers shared by the GPU parity tests: moving seeded numpy inputs to the
GPU in their storage dtype, reading results back exactly, and the error
metric the tolerances are stated in."""
import numpy as np

# Tolerances on err (below), per storage dtype; accumulation is fp32 throughout.
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to("cuda")


def to_host(t):
    """Exact float64 copy of a device tensor (f16/bf16/f32 widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref)): the RMS floor keeps
    outputs that cancel to near zero from dominating."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    denom = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / denom))


def say(*parts):
    """Name the case on stdout (flushed) before a GPU step."""
    print("[case]", *parts, flush=True)
