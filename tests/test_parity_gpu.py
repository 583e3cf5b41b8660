"""GPU parity: libdcn's HIP kernels against the CPU oracle, element by
element, on the same seeded inputs, at the workloads' full sizes and on edge
cases.  Bar: err <= 1e-5 for f32, <= 2e-2 for f16/bf16 (fp32 accumulation),
with err as defined in parity_util.rel_err."""
import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, say, to_dev, to_host
from sparse_deformable_sampling_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sds():
    import torch
    import sparse_deformable_sampling_amd as m
    assert torch.cuda.is_available()
    return m


def run_fwd(sds, d, dtype, group, softmax, **geom):
    x, off, mask = (to_dev(d[k], dtype) for k in ("x", "offset", "mask"))
    out = sds.dcn_forward(x, off, mask, group=group, softmax=softmax, **geom)
    return to_host(out)


def check_fwd(sds, name, n, h, w, c, g, dtype, softmax, offset=("normal", 1.5), seed=1, **geom):
    ho, wo = oracle.dcn_out_size(h, w, geom.get("kernel", 3), geom.get("stride", 1), geom.get("pad", 1),
                                 geom.get("dil", 1))
    assert sds.dcn_output_size(h, w, geom.get("kernel", 3), geom.get("stride", 1), geom.get("pad", 1),
                               geom.get("dil", 1)) == (ho, wo)
    kern = geom.get("kernel", 3)
    K = kern * kern if isinstance(kern, int) else kern[0] * kern[1]
    d = synth.dcn_inputs(n, h, w, c, g, (ho, wo), taps=K, offset=offset, dtype=dtype, seed=seed)
    say(name, dtype, "softmax=%d" % softmax, (n, h, w, c, g), geom)
    got = run_fwd(sds, d, dtype, g, softmax, **geom)
    ref = oracle.dcn_forward(d["x"], d["offset"], d["mask"], group=g, softmax=softmax, dtype=dtype, **geom)
    err = rel_err(got, ref)
    say("  err", name, dtype, "%.3e" % err)
    assert err <= TOL[dtype], (name, dtype, softmax, err)
    return err


# ---------------------------------------------------------------- forward


def test_dcnv3_tiny_f32(sds):
    """N=1 H=W=8 C=16 G=2, offsets U(-2,2), logits N(0,1) with softmax."""
    check_fwd(sds, "dcnv3-tiny", 1, 8, 8, 16, 2, "f32", True, offset=("uniform", -2.0, 2.0))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("softmax", [True, False])
def test_stage1_forward_full(sds, dtype, softmax):
    """InternImage-T stage-1 shape N=64 H=W=56 C=64 G=4, offsets N(0,1.5)."""
    check_fwd(sds, "stage1", 64, 56, 56, 64, 4, dtype, softmax)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("softmax", [False, True])
def test_table10_shape(sds, dtype, softmax):
    """The pages' module shape 56x56x128, 4 groups of 32 channels, at the
    benched batch of 64: a group is 128 bytes per pixel in f32 (64 in
    f16/bf16) and runs as four (two) 32-byte lane items sharing the group's
    offsets and mask."""
    check_fwd(sds, "table10", 64, 56, 56, 128, 4, dtype, softmax)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("softmax", [False, True])
def test_chunks_ending_in_a_partial_step(sds, dtype, softmax):
    """N=64, 50x56, C=64, G=4: every workgroup's chunk ends in a one-row
    step (f32: 25 rows, six steps of 4 and one of 1; f16/bf16: 13 rows,
    three of 4 and one of 1), so in the step before the last most lanes have
    an item and none in the next (their next-step offsets and mask are not
    loaded), and the last step runs a quarter full."""
    check_fwd(sds, "partial-step", 64, 50, 56, 64, 4, dtype, softmax, seed=23)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("stage", ["stage2", "stage3"])
def test_dcnv4_stage2_stage3_full(sds, dtype, stage):
    n, hw, c, g = {"stage2": (64, 28, 128, 8), "stage3": (64, 14, 320, 20)}[stage]
    check_fwd(sds, stage, n, hw, hw, c, g, dtype, False)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", ["9x9-g16", "27-stride2", "13x11-dcnv3", "wide-offsets", "13x13-ragged-chunks"])
def test_small_maps_many_images(sds, dtype, case):
    """Small maps in large batches, where a row chunk is most or all of an
    image and its halo reaches past the image on both sides: a 9x9 map with
    16 groups (batch 128); a 27x27 map at stride 2 (14x14 out, 20 groups); a
    ragged 13x11 map with the DCNv3 softmax (batch 256); offsets wide
    enough that many samples fall outside the image, above and below it; and
    a 13x13 map with 20 groups, whose chunks of one step each (two workgroups
    per CU) are 7 and 6 rows, with the DCNv3 softmax."""
    if case == "9x9-g16":
        check_fwd(sds, "small-map", 128, 9, 9, 256, 16, dtype, False, seed=31)
    elif case == "27-stride2":
        check_fwd(sds, "small-map", 64, 27, 27, 320, 20, dtype, False, seed=32, stride=2)
    elif case == "13x11-dcnv3":
        check_fwd(sds, "small-map", 256, 13, 11, 96, 6, dtype, True, seed=33)
    elif case == "wide-offsets":
        check_fwd(sds, "small-map", 64, 14, 14, 320, 20, dtype, False, offset=("normal", 6.0), seed=34)
    else:
        check_fwd(sds, "small-map", 64, 13, 13, 320, 20, dtype, True, seed=35)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c,g", [(4, 4), (12, 4), (15, 3), (16, 2), (32, 1), (64, 1), (256, 2), (24, 3), (512, 1),
                                 (1024, 2)])
def test_channel_splits(sds, dtype, c, g):
    """Every D = C/G path: one channel, odd D, D not a multiple of the vector
    width, vector widths exactly, several vectors per item, and groups of 512
    channels (split into up to 64 lane items of 32 bytes)."""
    for softmax in (False, True):
        check_fwd(sds, "split", 2, 9, 11, c, g, dtype, softmax, seed=3)


@pytest.mark.parametrize("geom", [dict(kernel=(3, 2), stride=(2, 1), pad=(1, 2), dil=(1, 2)),
                                  dict(kernel=1, stride=1, pad=0, dil=1),
                                  dict(kernel=5, stride=2, pad=2, dil=1),
                                  dict(kernel=3, stride=1, pad=0, dil=3),
                                  dict(kernel=(1, 7), stride=(1, 3), pad=(0, 3), dil=1),
                                  dict(kernel=3, stride=3, pad=1, dil=1)])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_geometries(sds, geom, dtype):
    for softmax in (False, True):
        check_fwd(sds, "geom", 2, 13, 10, 16, 2, dtype, softmax, seed=5, **geom)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_and_tiny_maps(sds, dtype):
    for (n, h, w) in [(1, 1, 1), (3, 1, 7), (1, 5, 1), (5, 3, 3), (7, 13, 17)]:
        check_fwd(sds, "ragged", n, h, w, 16, 2, dtype, False, seed=7)
        check_fwd(sds, "ragged", n, h, w, 16, 2, dtype, True, seed=7)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_offsets_far_outside_and_non_finite(sds, dtype):
    n, h, w, c, g = 2, 8, 9, 16, 2
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f32", seed=11)
    off = d["offset"].copy()
    rng = np.random.default_rng(0)
    pick = rng.random(off.shape) < 0.1
    off[pick] = rng.choice([1e6, -1e6, 3e4, -40.0, 8.5, -9.25], size=int(pick.sum()))
    off[0, 0, 0, 0, 0, 0] = np.inf
    off[0, 1, 1, 1, 3, 1] = -np.inf
    off[1, 2, 2, 0, 4, 0] = np.nan
    off[1, 3, 3, 1, 8, :] = [-1.0, -1.0]       # exactly on the edge
    d["offset"] = synth.store(off, dtype)
    d["x"] = synth.store(d["x"], dtype)
    d["mask"] = synth.store(d["mask"], dtype)
    for softmax in (False, True):
        say("outside", dtype, softmax)
        got = run_fwd(sds, d, dtype, g, softmax)
        ref = oracle.dcn_forward(d["x"], d["offset"], d["mask"], group=g, softmax=softmax, dtype=dtype)
        assert np.isfinite(got).all()
        assert rel_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c,g", [(64, 4), (32, 2), (24, 3), (15, 3)])
def test_non_finite_x_where_no_tap_reads(sds, dtype, c, g):
    """NaN and Inf in x at image column 0: an output whose taps never read a
    corner there must come out finite and equal to the oracle's, whether its
    other taps fall outside the map (they contribute exactly zero, so nothing
    may multiply those values by a zero weight), inside the on-chip window,
    or beyond it (|dy| up to 9); outputs that do read them are NaN/Inf in
    both."""
    n, h, w = 2, 20, 24
    rng = np.random.default_rng(97)
    x = rng.standard_normal((n, h, w, c)).astype(np.float32)
    x[:, :, 0, :] = np.nan
    x[:, ::3, 0, : c // 2] = np.inf
    x[:, 1::3, 0, c // 2:] = -np.inf
    # px = wo - 1 + kx + dx with dx in [0, 0.9): for wo >= 2 every corner
    # column is >= 1; dy spans +-9 rows.
    off = np.empty((n, h, w, g, 9, 2), np.float32)
    off[..., 0] = rng.uniform(0.0, 0.9, size=off.shape[:-1])
    off[..., 1] = np.clip(rng.normal(0.0, 3.0, size=off.shape[:-1]), -9.0, 9.0)
    far = rng.random(off.shape[:-1]) < 0.3
    off[..., 0][far] = rng.choice([-1000.0, 1000.0, -30.0], size=int(far.sum()))
    mask = rng.standard_normal((n, h, w, g, 9)).astype(np.float32)
    x, off, mask = (synth.store(a, dtype) for a in (x, off, mask))
    for softmax in (False, True):
        say("non-finite-x", dtype, (c, g), "softmax", softmax)
        out = sds.dcn_forward(to_dev(x, dtype), to_dev(off, dtype), to_dev(mask, dtype), group=g,
                              softmax=softmax)
        got = to_host(out)
        ref = oracle.dcn_forward(x, off, mask, group=g, softmax=softmax, dtype=dtype)
        fin = np.isfinite(ref)
        assert fin[:, :, 2:, :].all()   # the construction keeps these outputs clear of column 0
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        assert np.array_equal(np.isinf(got), np.isinf(ref))
        e = rel_err(got[fin], ref[fin])
        say("  err", "non-finite-x", dtype, "%.3e" % e)
        assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("std", [4.0, 12.0])
def test_wide_offsets_stage1(sds, dtype, std):
    """Offsets wide enough that many samples leave any row window kept
    on chip: every read path of the kernel, at the stage-1 shape."""
    for softmax in (False, True):
        check_fwd(sds, "wide-offsets", 16, 56, 56, 64, 4, dtype, softmax, offset=("normal", std), seed=23)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(3, 40, 9, 32, 2), (2, 7, 130, 16, 1), (5, 23, 5, 48, 3), (1, 3, 3, 64, 8)])
def test_tall_wide_and_short_maps(sds, dtype, shape):
    n, h, w, c, g = shape
    for softmax in (False, True):
        for geom in (dict(), dict(stride=2), dict(dil=2, pad=2)):
            check_fwd(sds, "shape", n, h, w, c, g, dtype, softmax, seed=29, **geom)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, 0.5, 2.0, -1.25])
def test_offset_scale(sds, dtype, scale):
    """offset_scale multiplies every offset before it is added (0 turns the
    op into a modulated sampling of the regular grid)."""
    for softmax in (False, True):
        check_fwd(sds, "offset-scale", 2, 14, 12, 32, 2, dtype, softmax, seed=61, offset_scale=scale)
    check_fwd(sds, "offset-scale", 4, 56, 56, 64, 4, dtype, False, seed=62, offset_scale=scale)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c,g", [(32, 2), (64, 4)])
def test_integer_offsets_bit_exact(sds, dtype, c, g):
    """One-hot DCNv4 modulation and integer offsets copy pixels exactly, in
    every storage type (the stored values are compared bit for bit)."""
    import torch
    n, h, w = 2, 10, 12
    rng = np.random.default_rng(13)
    x = synth.store(rng.standard_normal((n, h, w, c)).astype(np.float32), dtype)
    off = synth.store(rng.integers(-4, 5, size=(n, h, w, g, 9, 2)).astype(np.float32), dtype)
    mask = np.zeros((n, h, w, g, 9), np.float32)
    mask[..., 5] = 1.0
    mask = synth.store(mask, dtype)
    say("integer-shift", dtype, c, g)
    out = sds.dcn_forward(to_dev(x, dtype), to_dev(off, dtype), to_dev(mask, dtype), group=g)
    ref = oracle.dcn_forward(x, off, mask, group=g, dtype=dtype)
    got = to_host(out)
    assert np.array_equal(got, ref)
    torch.cuda.synchronize()


def test_unaligned_views_take_the_scalar_path(sds):
    """Tensors that start one element into an allocation are valid input."""
    import torch
    n, h, w, c, g = 2, 7, 6, 16, 2
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f32", seed=17)
    def shifted(a):
        t = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        v = t[1:].view(a.shape)
        v.copy_(torch.from_numpy(a))
        return v
    x, off, mask = shifted(d["x"]), shifted(d["offset"]), shifted(d["mask"])
    out = torch.empty(n * h * w * c + 1, device="cuda")[1:].view(n, h, w, c)
    say("unaligned")
    sds.dcn_forward(x, off, mask, group=g, out=out)
    ref = oracle.dcn_forward(d["x"], d["offset"], d["mask"], group=g)
    assert rel_err(to_host(out), ref) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_forward_is_deterministic(sds, dtype):
    import torch
    d = synth.dcn_inputs(8, 56, 56, 64, 4, (56, 56), dtype=dtype, seed=19)
    x, off, mask = (to_dev(d[k], dtype) for k in ("x", "offset", "mask"))
    say("determinism", dtype)
    a = sds.dcn_forward(x, off, mask, group=4)
    b = sds.dcn_forward(x, off, mask, group=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_invalid_call_leaves_output_untouched(sds):
    import torch
    from sparse_deformable_sampling_amd import _binding as B
    import ctypes
    x = torch.randn(1, 8, 8, 16, device="cuda")
    off = torch.zeros(1, 8, 8, 2, 9, 2, device="cuda")
    mask = torch.zeros(1, 8, 8, 2, 9, device="cuda")
    out = torch.full((1, 8, 8, 16), 7.0, device="cuda")
    desc = B.make_desc(1, 8, 8, 16, 3)   # 16 % 3 != 0
    st = B.lib().dcn_forward(ctypes.byref(desc), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(off.data_ptr()),
                             ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(out.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == B.DCN_ERR_INVALID
    assert bool((out == 7.0).all())
    with pytest.raises(B.DcnError):
        sds.dcn_forward(x, off[:, :, :, :1].contiguous(), mask[:, :, :, :1].contiguous(), group=3)


# ---------------------------------------------------------------- backward


def check_bwd(sds, name, n, h, w, c, g, softmax, seed=1, tol=None, offset=("normal", 1.5), gscale=1.0,
              dtype="f32", **geom):
    tol = TOL[dtype] if tol is None else tol
    kern = geom.get("kernel", 3)
    K = kern * kern if isinstance(kern, int) else kern[0] * kern[1]
    ho, wo = oracle.dcn_out_size(h, w, kern, geom.get("stride", 1), geom.get("pad", 1), geom.get("dil", 1))
    d = synth.dcn_inputs(n, h, w, c, g, (ho, wo), taps=K, offset=offset, dtype=dtype, seed=seed, grad=True)
    if gscale != 1.0:
        d["grad_out"] = synth.store(d["grad_out"] * np.float32(gscale), "f32")
    x, off, mask, go = (to_dev(d[k], dtype) for k in ("x", "offset", "mask", "grad_out"))
    say(name, dtype, "softmax=%d" % softmax, (n, h, w, c, g), geom)
    gx, goff, gm = sds.dcn_backward(x, off, mask, go, group=g, softmax=softmax, **geom)
    rx, roff, rm = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=g, softmax=softmax,
                                       dtype=dtype, **geom)
    errs = (rel_err(to_host(gx), rx), rel_err(to_host(goff), roff), rel_err(to_host(gm), rm))
    say("  err", name, dtype, "%.3e %.3e %.3e" % errs)
    assert max(errs) <= tol, (name, softmax, errs)
    return errs


@pytest.mark.parametrize("softmax", [True, False])
def test_backward_stage1_full(sds, softmax):
    """DCNv3 and DCNv4 backward, f32, N=64 H=W=56 C=64 G=4, grad_out N(0,1)."""
    check_bwd(sds, "bwd-stage1", 64, 56, 56, 64, 4, softmax)


@pytest.mark.parametrize("softmax", [True, False])
def test_backward_wide_offsets(sds, softmax):
    """Offsets N(0, 6): many corners land outside the rows a workgroup keeps
    on chip and take the direct path into grad_x."""
    check_bwd(sds, "bwd-wide", 8, 56, 56, 64, 4, softmax, seed=31, offset=("normal", 6.0))


@pytest.mark.parametrize("scale", [0.0, 0.5, 2.0, -1.25])
def test_backward_offset_scale(sds, scale):
    """grad_offset carries the factor offset_scale."""
    check_bwd(sds, "bwd-oscale", 4, 20, 24, 32, 2, False, seed=67, offset_scale=scale)
    check_bwd(sds, "bwd-oscale", 4, 20, 24, 32, 2, True, seed=67, offset_scale=scale)


@pytest.mark.parametrize("gscale", [1e-30, 1e-12, 1e12, 1e30])
def test_backward_gradient_scales(sds, gscale):
    """Output gradients scaled far from 1: the on-chip sums pick their scale
    from the data, or step aside when it is out of their range."""
    check_bwd(sds, "bwd-scale", 4, 20, 24, 32, 2, False, seed=37, gscale=gscale)
    check_bwd(sds, "bwd-scale", 4, 20, 24, 32, 2, True, seed=37, gscale=gscale)


@pytest.mark.parametrize("outliers", ["one-1e3", "one-1e4", "sparse-1e4", "dense-1e3"])
def test_backward_modulation_outliers(sds, outliers):
    """DCNv4 modulations are unbounded ("DCNv4: Unbounded Weights", "1. Remove
    Softmax"): a few very large mask values in otherwise N(0,1) stage-1
    planes (one value of 1e3 or 1e4 per image, one tap in a thousand at 1e4,
    or one in twenty at 1e3) must not coarsen the other sums of grad_x,
    which keep the f32 bar.  At this shape one workgroup covers a whole
    (image, group) plane."""
    import torch
    n, h, w, c, g = 64, 56, 56, 64, 4
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f32", seed=41, grad=True)
    mask = d["mask"].copy()
    rng = np.random.default_rng(43)
    if outliers.startswith("one"):
        v = 1e3 if outliers.endswith("1e3") else 1e4
        for i in range(n):   # one per image, in a random group and tap
            mask[i, rng.integers(h), rng.integers(w), rng.integers(g), rng.integers(9)] = v * rng.choice([-1, 1])
    else:
        frac, v = (1e-3, 1e4) if outliers.startswith("sparse") else (5e-2, 1e3)
        pick = rng.random(mask.shape) < frac
        mask[pick] = v * rng.choice([-1.0, 1.0], size=int(pick.sum()))
    d["mask"] = synth.store(mask, "f32")
    x, off, m, go = (to_dev(d[k], "f32") for k in ("x", "offset", "mask", "grad_out"))
    say("bwd-outliers", outliers)
    gx, goff, gm = sds.dcn_backward(x, off, m, go, group=g, softmax=False)
    torch.cuda.synchronize()
    rx, roff, rm = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=g, softmax=False)
    # grad_offset[k] = sigma * m_k * s_k, with s_k a channel sum of fp32 terms
    # that does not depend on m_k: its fp32 rounding scales with |m_k|, so an
    # element is measured against max(|r|, |m_k| * rms(r / m)), its own
    # natural scale, instead of the RMS of a tensor whose few huge taps
    # dominate the RMS while cancelling elements of those taps carry
    # |m_k| times an ordinary rounding.
    mk = np.abs(d["mask"].astype(np.float64))[..., None]
    scale = mk * np.sqrt(np.mean((roff / np.maximum(mk, 1e-30)) ** 2))
    e_off = float(np.max(np.abs(to_host(goff) - roff) / np.maximum(np.abs(roff), np.maximum(scale, 1e-30))))
    errs = (rel_err(to_host(gx), rx), e_off, rel_err(to_host(gm), rm))
    say("  err", "bwd-outliers", outliers, "x %.3e offset (own scale) %.3e mask %.3e" % errs,
        "offset (tensor rms) %.3e" % rel_err(to_host(goff), roff))
    assert max(errs) <= TOL["f32"], errs


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n,h,w", [(2, 20, 24), (64, 56, 56)])
def test_backward_non_finite_grad_out_and_mask(sds, dtype, n, h, w):
    """A few NaN and +-Inf values in grad_out and in the (DCNv4) mask: the
    gradients they reach are NaN/Inf as in the oracle, and every other
    element keeps the bar.  The fixed-point sums of grad_x choose their scale
    from a sample of the items, so a non-finite value outside the sample must
    still reach grad_x (through the fp32 atomics); (64, 56, 56) is the stage-1
    shape, where one workgroup covers a whole (image, group) plane."""
    import torch
    c, g = 64, 4
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f32", seed=47, grad=True)
    rng = np.random.default_rng(49)
    go, mask = d["grad_out"].copy(), d["mask"].copy()
    for arr, cnt in ((go, 6), (mask, 4)):
        flat = arr.reshape(-1)
        idx = rng.choice(flat.size, size=cnt, replace=False)
        flat[idx] = [np.nan, np.inf, -np.inf, np.nan, np.inf, -np.inf][:cnt]
    d["grad_out"], d["mask"] = go, mask
    for k in ("x", "offset", "mask", "grad_out"):
        d[k] = synth.store(d[k], dtype)
    say("bwd-non-finite", dtype, (n, h, w))
    outs = sds.dcn_backward(*(to_dev(d[k], dtype) for k in ("x", "offset", "mask", "grad_out")), group=g,
                            softmax=False)
    torch.cuda.synchronize()
    refs = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=g, softmax=False, dtype=dtype)
    for name, t, ref in zip(("grad_x", "grad_offset", "grad_mask"), outs, refs):
        got = to_host(t)
        # grad_x terms are m_k * w * g_c: zero in fp32 exactly when zero in
        # fp64, so NaN (0 * Inf) and +-Inf fall on the same elements.  A
        # grad_offset or grad_mask term multiplies g_c by a corner difference
        # or an interpolated value that can be exactly 0 in one precision and
        # tiny in the other, so there only the finite elements must agree
        # (NaN and Inf may trade places).
        if name == "grad_x":
            assert np.array_equal(np.isnan(got), np.isnan(ref)), name
            assert np.array_equal(np.isinf(got), np.isinf(ref)), name
            assert np.array_equal(np.signbit(got[np.isinf(ref)]), np.signbit(ref[np.isinf(ref)])), name
        assert np.array_equal(np.isfinite(got), np.isfinite(ref)), name
        fin = np.isfinite(ref)
        assert fin.mean() > 0.9, name
        e = rel_err(got[fin], ref[fin])
        say("  err", "bwd-non-finite", dtype, name, "%.3e" % e)
        assert e <= TOL[dtype], (name, e)


@pytest.mark.parametrize("softmax", [True, False])
def test_backward_crop_against_finite_differences(sds, softmax):
    """The 8x8 top-left crop of image 0 of the stage-1 inputs, as its own
    problem: GPU gradients against central differences of the oracle
    forward (double precision)."""
    d = synth.dcn_inputs(1, 56, 56, 64, 4, (56, 56), dtype="f32", seed=1, grad=True)
    x = np.ascontiguousarray(d["x"][:, :8, :8])
    off = np.ascontiguousarray(d["offset"][:, :8, :8])
    mask = np.ascontiguousarray(d["mask"][:, :8, :8])
    go = np.ascontiguousarray(d["grad_out"][:, :8, :8])
    say("bwd-crop-fd", softmax)
    gx, goff, gm = sds.dcn_backward(to_dev(x, "f32"), to_dev(off, "f32"), to_dev(mask, "f32"), to_dev(go, "f32"),
                                    group=4, softmax=softmax)
    gx, goff, gm = to_host(gx), to_host(goff), to_host(gm)
    rx, roff, rm = oracle.dcn_backward(x, off, mask, go, group=4, softmax=softmax)
    assert max(rel_err(gx, rx), rel_err(goff, roff), rel_err(gm, rm)) <= TOL["f32"]

    x64, off64, m64, go64 = (a.astype(np.float64) for a in (x, off, mask, go))

    def loss(xx, oo, mm):
        return float(np.sum(go64 * oracle.dcn_forward(xx, oo, mm, group=4, softmax=softmax)))

    h = 1e-6
    rng = np.random.default_rng(23)
    checked = 0
    for _ in range(40):
        ix = tuple(int(rng.integers(0, s)) for s in off.shape)
        yo, xo, kk, comp = ix[1], ix[2], ix[4], ix[5]
        coord = (xo - 1 + kk // 3 if comp == 0 else yo - 1 + kk % 3) + off64[ix]
        if abs(coord - round(coord)) < 1e-4:
            continue
        a, b = off64.copy(), off64.copy()
        a[ix] += h
        b[ix] -= h
        fd = (loss(x64, a, m64) - loss(x64, b, m64)) / (2 * h)
        assert goff[ix] == pytest.approx(fd, rel=1e-4, abs=1e-4)
        checked += 1
    assert checked >= 30
    for _ in range(20):
        ix = tuple(int(rng.integers(0, s)) for s in mask.shape)
        a, b = m64.copy(), m64.copy()
        a[ix] += h
        b[ix] -= h
        fd = (loss(x64, off64, a) - loss(x64, off64, b)) / (2 * h)
        assert gm[ix] == pytest.approx(fd, rel=1e-4, abs=1e-4)
    for _ in range(20):
        ix = tuple(int(rng.integers(0, s)) for s in x.shape)
        a, b = x64.copy(), x64.copy()
        a[ix] += h
        b[ix] -= h
        fd = (loss(a, off64, m64) - loss(b, off64, m64)) / (2 * h)
        assert gx[ix] == pytest.approx(fd, rel=1e-4, abs=1e-4)


@pytest.mark.parametrize("c,g", [(16, 4), (12, 4), (15, 3), (32, 1), (256, 2), (8, 8), (48, 2), (512, 1)])
def test_backward_channel_splits(sds, c, g):
    for softmax in (False, True):
        check_bwd(sds, "bwd-split", 2, 9, 11, c, g, softmax, seed=29)


@pytest.mark.parametrize("geom", [dict(kernel=(3, 2), stride=(2, 1), pad=(1, 2), dil=(1, 2)),
                                  dict(kernel=5, stride=2, pad=2, dil=1),
                                  dict(kernel=1, stride=1, pad=0, dil=1)])
def test_backward_geometries(sds, geom):
    for softmax in (False, True):
        check_bwd(sds, "bwd-geom", 2, 13, 10, 16, 2, softmax, seed=31, **geom)


# ---------------------------------------------------------------- half-precision backward

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("softmax", [True, False])
def test_backward_half_stage1_full(sds, dtype, softmax):
    """f16/bf16 backward at N=64 H=W=56 C=64 G=4: inputs and grads in the
    half type, fp32 arithmetic, grad_x summed in an fp32 workspace."""
    check_bwd(sds, "bwd-half-stage1", 64, 56, 56, 64, 4, softmax, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("stage", ["stage2", "stage3"])
def test_backward_half_stage2_stage3(sds, dtype, stage):
    n, hw, c, g = {"stage2": (64, 28, 128, 8), "stage3": (64, 14, 320, 20)}[stage]
    check_bwd(sds, "bwd-half-" + stage, n, hw, hw, c, g, False, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c,g", [(16, 4), (12, 4), (15, 3), (32, 1), (8, 4), (48, 2), (2, 1)])
def test_backward_half_channel_splits(sds, dtype, c, g):
    """D = 4, 3, 5, 32, 2, 24, 2: the windowed kernel with 4 or 8 channels
    per lane (8- and 16-byte gathers of 16-bit values), the lane-per-channel
    and the generic fallbacks."""
    for softmax in (False, True):
        check_bwd(sds, "bwd-half-split", 2, 9, 11, c, g, softmax, seed=71, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_half_wide_offsets_and_geometries(sds, dtype):
    check_bwd(sds, "bwd-half-wide", 4, 40, 44, 64, 4, True, seed=73, offset=("normal", 6.0), dtype=dtype)
    check_bwd(sds, "bwd-half-geom", 2, 13, 10, 16, 2, False, seed=79, dtype=dtype,
              kernel=(3, 2), stride=(2, 1), pad=(1, 2), dil=(1, 2))
    check_bwd(sds, "bwd-half-oscale", 2, 12, 14, 32, 2, False, seed=83, dtype=dtype, offset_scale=-1.25)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_half_partial_outputs(sds, dtype):
    """Without grad_x no workspace is used; grad_x alone still matches."""
    d = synth.dcn_inputs(2, 9, 9, 16, 2, (9, 9), dtype=dtype, seed=89, grad=True)
    x, off, mask, go = (to_dev(d[k], dtype) for k in ("x", "offset", "mask", "grad_out"))
    say("bwd-half-partial", dtype)
    rx, roff, rm = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=2, dtype=dtype)
    gx, goff, gm = sds.dcn_backward(x, off, mask, go, group=2, need_x=False)
    assert gx is None and rel_err(to_host(goff), roff) <= TOL[dtype] and rel_err(to_host(gm), rm) <= TOL[dtype]
    gx, goff, gm = sds.dcn_backward(x, off, mask, go, group=2, need_offset=False, need_mask=False)
    assert goff is None and gm is None and rel_err(to_host(gx), rx) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_backward_samples_exactly_on_the_lower_edges(sds, dtype):
    """Integer offsets that put samples exactly at px = -1 or py = -1: such a
    sample is outside the map (zero value and zero gradient), while samples
    at other integer coordinates take the right-hand derivative."""
    n, h, w, c, g = 2, 7, 9, 16, 2
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f32", seed=97, grad=True)
    off = d["offset"].copy()                      # [n, ho, wo, g, 9, 2], tap k = kx*3 + ky
    off[:, :, 0, :, 0:3, 0] = 0.0                 # wo = 0, kx = 0: px = -1 exactly
    off[:, 0, :, :, 0::3, 1] = 0.0                # ho = 0, ky = 0: py = -1 exactly
    off[:, :, 1, :, 0:3, 0] = -1.0                # wo = 1, kx = 0: px = -1 again
    off[:, 3, :, :, 3:6, 0] = np.float32(2.0)     # an interior integer coordinate
    d["offset"] = off
    if dtype != "f32":
        d = {k: synth.store(v.astype(np.float32), dtype) for k, v in d.items()}
    x, o, m, go = (to_dev(d[k], dtype) for k in ("x", "offset", "mask", "grad_out"))
    say("bwd-edges", dtype)
    for softmax in (False, True):
        gx, goff, gm = sds.dcn_backward(x, o, m, go, group=g, softmax=softmax)
        rx, roff, rm = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=g,
                                           softmax=softmax, dtype=dtype)
        errs = (rel_err(to_host(gx), rx), rel_err(to_host(goff), roff), rel_err(to_host(gm), rm))
        assert max(errs) <= TOL[dtype], (dtype, softmax, errs)
        assert np.all(to_host(goff)[:, :, 0, :, 0:3, 0] == 0.0)


def test_backward_partial_outputs(sds):
    d = synth.dcn_inputs(2, 9, 9, 16, 2, (9, 9), dtype="f32", seed=37, grad=True)
    x, off, mask, go = (to_dev(d[k], "f32") for k in ("x", "offset", "mask", "grad_out"))
    say("bwd-partial")
    rx, roff, rm = oracle.dcn_backward(d["x"], d["offset"], d["mask"], d["grad_out"], group=2)
    gx, goff, gm = sds.dcn_backward(x, off, mask, go, group=2, need_x=False)
    assert gx is None and rel_err(to_host(goff), roff) <= 1e-5 and rel_err(to_host(gm), rm) <= 1e-5
    gx, goff, gm = sds.dcn_backward(x, off, mask, go, group=2, need_offset=False, need_mask=False)
    assert goff is None and gm is None and rel_err(to_host(gx), rx) <= 1e-5


# ---------------------------------------------------------------- MSDA

ENCODER_SHAPES = [(100, 134), (50, 67), (25, 34), (13, 17)]


def check_msda(sds, name, n, shapes, q, heads, dh, points, softmax=True, seed=1, offset_std=2.0, ref="uniform"):
    d = synth.msda_inputs(n, shapes, q, heads, dh, points, offset_std=offset_std, seed=seed, ref=ref)
    v, loc, attn = (to_dev(d[k], "f32") for k in ("value", "loc", "attn"))
    say(name, (n, shapes, q, heads, dh, points), softmax)
    got = to_host(sds.msda_forward(v, shapes, loc, attn, softmax=softmax))
    ref = oracle.msda_forward(d["value"], shapes, d["loc"], d["attn"], softmax=softmax)
    err = rel_err(got, ref)
    assert err <= TOL["f32"], (name, err)
    return err


@pytest.mark.parametrize("ref", ["cells", "uniform"])
def test_msda_encoder_full(sds, ref):
    """Batch 8, 4 levels (100x134 .. 13x17), all 17821 positions as queries,
    8 heads x 32, 4 points per level, joint softmax over 16; reference points
    at the queries' own cell centres (the encoder) or uniform at random."""
    check_msda(sds, "msda-encoder-" + ref, 8, ENCODER_SHAPES, 17821, 8, 32, 4, ref=ref)


@pytest.mark.parametrize("dh", [1, 3, 4, 8, 32, 64, 36])
def test_msda_head_dims(sds, dh):
    check_msda(sds, "msda-dh", 2, [(7, 9), (4, 5)], 23, 3, dh, 3, seed=41)


@pytest.mark.parametrize("n,shapes,q,heads,dh,points", [
    (2, [(6, 5), (3, 3)], 77, 3, 4, 8),          # 16 samples, one channel chunk per query
    (2, [(9, 7), (5, 4)], 50, 5, 64, 2),         # 4 samples, 16 lanes per query
    (1, [(4, 4)], 9, 1, 256, 32),                # 32 samples, 64 lanes per query
    (3, [(7, 6), (4, 3), (2, 2), (1, 1)], 45, 2, 16, 8),   # 32 samples over 4 levels
    (1, [(3, 3)], 40, 2, 4, 32),                 # a 32-lane workgroup
    (2, [(5, 8)], 300, 3, 8, 1),                 # one sample per head
])
def test_msda_tiled_shapes(sds, n, shapes, q, heads, dh, points):
    """Power-of-two sample counts and head sizes (the tiled kernel): ragged
    query tiles and workgroup counts that are not a multiple of eight."""
    for softmax in (True, False):
        check_msda(sds, "msda-tiled", n, shapes, q, heads, dh, points, softmax=softmax, seed=47, offset_std=3.0)


MID_SHAPES = [(64, 80), (32, 40), (16, 20), (8, 10)]   # S = 6800


@pytest.mark.parametrize("q,dh,points,softmax,ref", [
    (6800, 32, 4, True, "cells"),      # the encoder recipe at a third of its cells
    (6000, 32, 4, False, "uniform"),   # a ragged last tile, raw weights, random locations
    (3400, 64, 2, True, "uniform"),    # 16 lanes per query
    (6800, 16, 4, True, "cells"),      # 4 lanes per query
])
def test_msda_mid_size(sds, q, dh, points, softmax, ref):
    """Mid-size MSDA (2 images, 8 heads, thousands of queries over 4 levels):
    many tiles per (image, head) pair, every tile kind of the tiled kernel."""
    check_msda(sds, "msda-mid", 2, MID_SHAPES, q, 8, dh, points, softmax=softmax, seed=43, ref=ref)


SIXTEEN_LEVELS = [(i % 5 + 1, i % 3 + 2) for i in range(16)]   # the most levels the library takes


@pytest.mark.parametrize("shapes,points", [([(1, 1)], 1), ([(5, 3)], 8), ([(9, 7), (5, 4), (3, 2), (2, 1), (1, 1)], 2),
                                           (SIXTEEN_LEVELS, 2)])
def test_msda_levels_points(sds, shapes, points):
    for softmax in (True, False):
        check_msda(sds, "msda-lp", 2, shapes, 17, 2, 8, points, softmax=softmax, seed=43, offset_std=4.0)


# ---------------------------------------------------------------- MSDA from references (NEXT-4)

def check_msda_ref(sds, name, n, shapes, q, heads, dh, points, ref_dims, padded=True, softmax=True, seed=1,
                   ref="uniform"):
    import torch
    d = synth.msda_ref_inputs(n, shapes, q, heads, dh, points, ref_dims=ref_dims, padded=padded, seed=seed, ref=ref)
    v, ref, off, attn = (to_dev(d[k], "f32") for k in ("value", "reference", "offsets", "attn"))
    ratios = to_dev(d["valid_ratios"], "f32") if padded else None
    pad = torch.from_numpy(d["padding_mask"]).cuda() if padded else None
    say(name, (n, shapes, q, heads, dh, points), "ref_dims=%d padded=%d softmax=%d" % (ref_dims, padded, softmax))
    got = to_host(sds.msda_forward_ref(v, shapes, ref, off, attn, valid_ratios=ratios, padding_mask=pad,
                                       softmax=softmax))
    want = oracle.msda_forward_ref(d["value"], shapes, d["reference"], d["offsets"], d["attn"],
                                   d["valid_ratios"], d["padding_mask"], softmax=softmax)
    err = rel_err(got, want)
    say("  err", name, "%.3e" % err)
    assert err <= TOL["f32"], (name, err)


@pytest.mark.parametrize("ref", ["uniform", "cells"])
def test_msda_ref_encoder_padded(sds, ref):
    """Encoder shape (batch 8, 4 levels 100x134 .. 13x17, 8 heads x 32,
    4 points), point references, per-image valid ratios and padding: random
    references, and every cell a query referring to its own centre in the
    valid frame (the encoder's reference points, the benched workload)."""
    check_msda_ref(sds, "msda-ref-encoder-" + ref, 8, ENCODER_SHAPES, 17821, 8, 32, 4, 2, ref=ref)


@pytest.mark.parametrize("padded", [True, False])
@pytest.mark.parametrize("softmax", [True, False])
def test_msda_ref_decoder_boxes(sds, padded, softmax):
    """Decoder-like: 300 box references per image over the encoder levels."""
    check_msda_ref(sds, "msda-ref-boxes", 4, ENCODER_SHAPES, 300, 8, 32, 4, 4, padded=padded, softmax=softmax,
                   seed=61)


@pytest.mark.parametrize("ref_dims", [2, 4])
@pytest.mark.parametrize("n,shapes,q,heads,dh,points", [
    (2, [(6, 5), (3, 3)], 77, 3, 4, 8),              # tiled kernel
    (1, [(4, 4)], 9, 1, 256, 32),                     # tiled, 64 lanes per query
    (2, [(7, 9), (4, 5)], 23, 3, 36, 3),              # vec4 kernel (6 samples)
    (2, [(9, 7), (5, 4), (3, 2)], 17, 2, 3, 2),       # generic kernel (head_dim 3)
])
def test_msda_ref_shapes(sds, ref_dims, n, shapes, q, heads, dh, points):
    for padded in (True, False):
        check_msda_ref(sds, "msda-ref", n, shapes, q, heads, dh, points, ref_dims, padded=padded, seed=67)


def test_msda_ref_matches_loc_path(sds):
    """With ratios of 1 and no mask, the in-kernel locations give the same
    result as msda_forward at the oracle's locations (f32-rounded)."""
    shapes = [(6, 5), (3, 3)]
    d = synth.msda_ref_inputs(2, shapes, 40, 2, 8, 4, ref_dims=2, padded=False, seed=71)
    loc = oracle.msda_locations(d["reference"], d["offsets"], shapes).astype(np.float32)
    v, ref, off, attn, lc = (to_dev(a, "f32") for a in (d["value"], d["reference"], d["offsets"], d["attn"], loc))
    say("msda-ref-vs-loc")
    a = to_host(sds.msda_forward_ref(v, shapes, ref, off, attn))
    b = to_host(sds.msda_forward(v, shapes, lc, attn))
    assert rel_err(a, b) <= TOL["f32"]


# ---------------------------------------------------------------- MSDA backward


# Bars for (grad_value, grad_loc, grad_attn).  The gather path sums each
# cell's terms in fp64 and rounds once, so every output keeps the f32 bar.
# The atomic scatter adds its terms to grad_value in fp32, one per (query,
# sample, corner) that lands on the cell, in run-dependent order; at the
# encoder shape a cell of the 13x17 level takes about 17821*4*4/221 ~ 1300
# of them per head, and the round-off of a k-term fp32 sum is bounded by about
# k * 2^-24 of the sum of the terms' magnitudes (~8e-5 for k = 1300), hence a
# 1e-4 bar for that one output of that one path.
MSDA_BWD_TOL_GATHER = (TOL["f32"], TOL["f32"], TOL["f32"])
MSDA_BWD_TOL_ATOMIC = (1e-4, TOL["f32"], TOL["f32"])


def has_gather_path(n, shapes, q, heads, dh, points):
    """Whether msda_backward_ws gathers grad_value for this shape (a nonzero
    workspace size); otherwise it scatters with fp32 atomics like msda_backward."""
    import ctypes
    from sparse_deformable_sampling_amd import _binding as B
    desc = B.MsdaDesc(n, q, heads, dh, len(shapes), points, 1, B.DCN_F32)
    shp = (ctypes.c_int32 * (2 * len(shapes)))(*[v for hw in shapes for v in hw])
    nb = ctypes.c_size_t(0)
    assert B.lib().msda_backward_workspace_size(ctypes.byref(desc), shp, ctypes.byref(nb)) == B.DCN_OK
    return nb.value > 0


def msda_bwd_tol(gather, shape=None):
    """The bars of the path that runs: `gather` asks for the gather path, which
    `shape` (n, shapes, q, heads, dh, points) may not have."""
    if gather and (shape is None or has_gather_path(*shape)):
        return MSDA_BWD_TOL_GATHER
    return MSDA_BWD_TOL_ATOMIC


def check_msda_bwd(sds, name, n, shapes, q, heads, dh, points, softmax=True, seed=1, offset_std=2.0, ref="uniform"):
    import torch
    d = synth.msda_inputs(n, shapes, q, heads, dh, points, offset_std=offset_std, seed=seed, ref=ref)
    g = synth.store(np.random.default_rng(seed + 1000).standard_normal((n, q, heads, dh)).astype(np.float32), "f32")
    v, loc, attn, go = (to_dev(a, "f32") for a in (d["value"], d["loc"], d["attn"], g))
    rv, rl, ra = oracle.msda_backward(d["value"], shapes, d["loc"], d["attn"], g, softmax=softmax)
    errs = []
    for gather in (True, False):   # grad_value gathered per cell / scattered with atomics
        say(name, (n, shapes, q, heads, dh, points), "softmax", softmax, "gather", gather)
        gv, gl, ga = sds.msda_backward(v, shapes, loc, attn, go, softmax=softmax, gather=gather)
        torch.cuda.synchronize()
        e = (rel_err(to_host(gv), rv), rel_err(to_host(gl), rl), rel_err(to_host(ga), ra))
        tol = msda_bwd_tol(gather, (n, shapes, q, heads, dh, points))
        path = "gather" if tol is MSDA_BWD_TOL_GATHER else "atomic"
        say("  err", name, path, "value %.3e loc %.3e attn %.3e" % e)
        assert all(x <= t for x, t in zip(e, tol)), (name, softmax, gather, path, e)
        errs.append(e)
    return errs


@pytest.mark.parametrize("softmax,ref", [(True, "cells"), (False, "cells"), (True, "uniform")])
def test_msda_backward_encoder_full(sds, softmax, ref):
    """Batch 8, 4 levels (100x134 .. 13x17), all 17821 positions as queries,
    8 heads x 32, 4 points per level; reference points at the queries' own
    cell centres (the encoder) or uniform at random."""
    check_msda_bwd(sds, "msda-bwd-encoder-" + ref, 8, ENCODER_SHAPES, 17821, 8, 32, 4, softmax=softmax, ref=ref)


@pytest.mark.parametrize("n,shapes,q,heads,dh,points", [
    (2, [(6, 5), (3, 3)], 77, 3, 4, 8),          # tiled: 16 samples, 4 lanes per query
    (2, [(9, 7), (5, 4)], 50, 5, 64, 2),         # tiled: 64 lanes per query
    (1, [(4, 4)], 9, 1, 1, 32),                  # tiled: one channel, 32 samples
    (3, [(7, 6), (4, 3), (2, 2), (1, 1)], 45, 2, 16, 8),
    (1, [(5, 4), (3, 3)], 60, 2, 4, 16),         # 32 samples, one lane per query: 32 queries per workgroup
    (2, [(i % 5 + 1, i % 3 + 2) for i in range(16)], 40, 2, 8, 1),   # 16 levels, one point each
    (2, [(7, 9), (4, 5)], 23, 3, 36, 3),         # generic: 6 samples, head_dim 36
    (2, [(9, 7), (5, 4), (3, 2), (2, 1), (1, 1)], 17, 2, 8, 2),   # generic: 10 samples
])
def test_msda_backward_shapes(sds, n, shapes, q, heads, dh, points):
    for softmax in (True, False):
        check_msda_bwd(sds, "msda-bwd", n, shapes, q, heads, dh, points, softmax=softmax, seed=53, offset_std=3.0)


@pytest.mark.parametrize("dh,q,shapes", [
    (4, 700, [(5, 9), (2, 3)]),       # one lane per cell block; 64 groups per block on the 2x3 level
    (8, 600, [(6, 5), (1, 1)]),       # a 1x1 level: every sample shares the four buckets around it
    (16, 900, [(5, 4), (2, 2)]),
    (64, 500, [(7, 6), (3, 2)]),      # 16 lanes per block, up to 16 groups per block
])
def test_msda_backward_gather_many_samples_per_cell(sds, dh, q, shapes):
    """Gather path with head_dim 4..64 and levels small enough that a block
    of cells is split over several lane groups (summed through LDS), against
    the oracle and the atomic scatter."""
    check_msda_bwd(sds, "msda-bwd-split", 2, shapes, q, 2, dh, 2, softmax=True, seed=67, offset_std=1.0)


def test_msda_backward_crowded_cells(sds):
    """Every sample of an (image, head) pair in one bucket per level: the
    gather's runs are thousands of records long (len_q * points per level),
    against the oracle and the atomic scatter; a second pair reads nothing
    inside (all samples far outside), so its grad_value must come back zero.
    Four levels of two points: 8 samples per head, a shape with a gather
    path."""
    import torch
    shapes = [(12, 10), (6, 5), (3, 3), (2, 2)]
    n, q, heads, dh, points = 1, 1500, 2, 32, 2
    assert has_gather_path(n, shapes, q, heads, dh, points)
    d = synth.msda_inputs(n, shapes, q, heads, dh, points, seed=61)
    loc = d["loc"].copy()
    loc[0, :, 0] = [0.43, 0.57]          # head 0: one point on every level
    loc[0, :, 1] = [-3.0, 0.5]           # head 1: outside everywhere
    d["loc"] = synth.store(loc, "f32")
    g = synth.store(np.random.default_rng(7).standard_normal((n, q, heads, dh)).astype(np.float32), "f32")
    v, lc, at, go = (to_dev(a, "f32") for a in (d["value"], d["loc"], d["attn"], g))
    rv, rl, ra = oracle.msda_backward(d["value"], shapes, d["loc"], d["attn"], g, softmax=True)
    for gather in (True, False):
        say("msda-bwd-crowded", "gather", gather)
        got = sds.msda_backward(v, shapes, lc, at, go, gather=gather)
        torch.cuda.synchronize()
        tols = msda_bwd_tol(gather, (n, shapes, q, heads, dh, points))
        for t, ref, tol in zip(got, (rv, rl, ra), tols):
            e = rel_err(to_host(t), ref)
            say("  err", "msda-bwd-crowded", "gather" if tols is MSDA_BWD_TOL_GATHER else "atomic", "%.3e" % e)
            assert e <= tol, gather
        assert np.all(to_host(got[0])[0, :, 1] == 0.0)


def test_msda_backward_far_outside_and_partial_outputs(sds):
    import torch
    shapes = [(6, 5), (3, 4)]
    n, q, heads, dh, points = 2, 33, 2, 8, 4
    d = synth.msda_inputs(n, shapes, q, heads, dh, points, seed=59)
    loc = d["loc"].copy()
    loc[0, 3, 1, 0, 2] = [-2.5, 0.5]
    loc[1, 7, 0, 1, 1] = [0.5, 3.0]
    loc[1, 8, 1, 1, 3] = [1.0 + 0.5 / 4, 0.5]     # x exactly at W: outside
    d["loc"] = synth.store(loc, "f32")
    g = synth.store(np.random.default_rng(5).standard_normal((n, q, heads, dh)).astype(np.float32), "f32")
    v, lc, at, go = (to_dev(a, "f32") for a in (d["value"], d["loc"], d["attn"], g))
    rv, rl, ra = oracle.msda_backward(d["value"], shapes, d["loc"], d["attn"], g, softmax=True)
    for gather in (True, False):
        say("msda-bwd-partial", "gather", gather)
        full = sds.msda_backward(v, shapes, lc, at, go, gather=gather)
        torch.cuda.synchronize()
        tols = msda_bwd_tol(gather, (n, shapes, q, heads, dh, points))
        for got, ref, tol in zip(full, (rv, rl, ra), tols):
            assert rel_err(to_host(got), ref) <= tol
        assert np.all(to_host(full[1])[0, 3, 1, 0, 2] == 0.0)
        for need in [(True, False, False), (False, True, False), (False, False, True)]:
            got = sds.msda_backward(v, shapes, lc, at, go, need_value=need[0], need_loc=need[1], need_attn=need[2],
                                    gather=gather)
            torch.cuda.synchronize()
            for flag, t, ref, tol in zip(need, got, (rv, rl, ra), tols):
                if flag:
                    assert rel_err(to_host(t), ref) <= tol
                else:
                    assert t is None


# ---------------------------------------------------------------- DCNv4 front-end


FRONT_KEYS = ("x", "dw_weight", "dw_bias", "om_weight", "om_bias")


def check_frontend(sds, name, n, h, w, c, g, dtype, kernel=3, dil=1, seed=1):
    kh, kw = (kernel, kernel) if isinstance(kernel, int) else kernel
    K = kh * kw
    d = synth.frontend_inputs(n, h, w, c, g, taps=K, dtype=dtype, seed=seed)
    say(name, dtype, (n, h, w, c, g), "kernel", kernel, "dil", dil)
    off, mask = sds.dcnv4_offset_mask(*(to_dev(d[k], dtype) for k in FRONT_KEYS), group=g, kernel=kernel, dil=dil)
    roff, rmask = oracle.dcnv4_offset_mask(*(d[k] for k in FRONT_KEYS), group=g, taps=K, dtype=dtype)
    eo, em = rel_err(to_host(off), roff), rel_err(to_host(mask), rmask)
    say("  err", name, dtype, "offset %.3e mask %.3e" % (eo, em))
    assert eo <= TOL[dtype] and em <= TOL[dtype], (name, dtype, eo, em)
    return d, off, mask


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("stage", ["stage1", "stage2", "stage3", "table10"])
def test_frontend_stages_full(sds, dtype, stage):
    """The DCNv4 front-end at the three stage shapes (C=64/128/320, G=4/8/20)
    and the pages' module shape (56x56x128, G=4), at the benched batch of 64
    (the wave kernel for C=64/128, the tile kernel for C=320)."""
    n, hw, c, g = {"stage1": (64, 56, 64, 4), "stage2": (64, 28, 128, 8), "stage3": (64, 14, 320, 20),
                   "table10": (64, 56, 128, 4)}[stage]
    check_frontend(sds, stage, n, hw, hw, c, g, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_frontend_one_block_per_wave(sds, dtype):
    """N=48, 28x28x128, G=8: 2352 blocks of 16 pixels, between 8 and 16 per
    CU, so the launch gives each CU one workgroup with a wave per block (10
    waves, 240 workgroups for 2352 blocks: the last ones short)."""
    check_frontend(sds, "one-block", 48, 28, 28, 128, 8, dtype, seed=41)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 8, 1), (2, 3, 70, 8, 2), (1, 5, 129, 24, 3), (3, 9, 11, 40, 5),
                                   (1, 2, 64, 136, 1), (1, 4, 65, 16, 16), (1, 7, 3, 512, 8), (1, 3, 10, 64, 2),
                                   (2, 6, 20, 256, 4), (1, 5, 7, 192, 2), (2, 4, 9, 256, 8),
                                   (1, 5, 7, 160, 10)])
def test_frontend_ragged_shapes(sds, dtype, shape):
    """Blocks cut mid-row and at the end of the data (870, 645, 30 pixels),
    odd widths (one-pixel runs), one pixel, C not a multiple of 32 (8, 24, 40,
    136: the zero-padded k tail), C = 256 (the widest wave-kernel case), C =
    136, 160, 192 and 512 (the tile kernel; 160 with 270 outputs on one
    ragged tile), output counts not a multiple of 16 or of 4 per pixel
    (3*9*g), 432 outputs."""
    n, h, w, c, g = shape
    check_frontend(sds, "ragged", n, h, w, c, g, dtype, seed=31)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_frontend_other_kernels(sds, dtype):
    """K = kernel_h*kernel_w outputs per group for other same-size kernels
    (the depthwise stays 3x3)."""
    check_frontend(sds, "k5", 2, 9, 10, 32, 2, dtype, kernel=5)
    check_frontend(sds, "k1x3", 2, 9, 10, 32, 4, dtype, kernel=(1, 3))
    check_frontend(sds, "k3d2", 2, 9, 10, 32, 2, dtype, kernel=3, dil=2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_frontend_feeds_the_core(sds, dtype):
    """Front-end then core op, both on the GPU, against the oracle's front-end
    then its core op.  The inputs make every depthwise sum and every offset
    and mask value exactly representable in the storage type (see
    synth.frontend_exact_inputs), so the chain has no rounding between its
    halves and the layouts the front-end writes must be the ones the core
    reads, value for value.  (With N(0,1) inputs each half meets its bar on
    its own, but an offset that rounds to the neighbouring f16/bf16 value on
    one side and not the other moves a sample by one unit in the last place,
    which the core's output can amplify past the bar.)"""
    n, h, w, c, g = 2, 12, 13, 64, 4
    d = synth.frontend_exact_inputs(n, h, w, c, g, dtype=dtype, seed=37)
    value = synth.module_inputs(n, h, w, c, g, dtype=dtype, seed=37)["value"]
    off, mask = sds.dcnv4_offset_mask(*(to_dev(d[k], dtype) for k in FRONT_KEYS), group=g)
    roff, rmask = oracle.dcnv4_offset_mask(*(d[k] for k in FRONT_KEYS), group=g, dtype=dtype)
    assert np.array_equal(to_host(off).astype(np.float64), roff)
    assert np.array_equal(to_host(mask).astype(np.float64), rmask)
    out = sds.dcn_forward(to_dev(value, dtype), off, mask, group=g, softmax=False)
    ref = oracle.dcn_forward(value, roff, rmask, group=g, softmax=False)
    err = rel_err(to_host(out), ref)
    say("  err chain core", dtype, "%.3e" % err)
    assert err <= TOL[dtype]


# ---------------------------------------------------------------- streams


def test_ops_follow_the_current_stream(sds):
    """Every wrapper enqueues on torch's current stream.  Inputs are produced
    on a side stream (of default priority), the ops run on it, and only that
    stream is waited for: a kernel launched elsewhere would race the copies.
    Results must equal those of the default stream (the forward bit for bit,
    the backward within the bars, its atomics being order-dependent)."""
    import torch
    n, h, w, c, g = 4, 20, 24, 64, 4
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f16", seed=71)
    fe = synth.frontend_inputs(n, h, w, c, g, dtype="f16", seed=72)
    go = synth.store(np.random.default_rng(73).standard_normal((n, h, w, c)).astype(np.float32), "f16")
    shapes = [(12, 10), (6, 5)]
    m = synth.msda_inputs(2, shapes, 150, 4, 32, 4, seed=74)
    mg = np.random.default_rng(75).standard_normal((2, 150, 4, 32)).astype(np.float32)
    base = {k: to_dev(d[k], "f16") for k in ("x", "offset", "mask")}
    base.update({"go": to_dev(go, "f16"), "v": to_dev(m["value"], "f32"), "loc": to_dev(m["loc"], "f32"),
                 "attn": to_dev(m["attn"], "f32"), "mg": to_dev(mg, "f32")})
    base.update({"fe_" + k: to_dev(fe[k], "f16") for k in FRONT_KEYS})
    torch.cuda.synchronize()

    def run(t):
        out = {"fwd": sds.dcn_forward(t["x"], t["offset"], t["mask"], group=g)}
        out["bwd"] = sds.dcn_backward(t["x"], t["offset"], t["mask"], t["go"], group=g)
        out["om"] = sds.dcnv4_offset_mask(*(t["fe_" + k] for k in FRONT_KEYS), group=g)
        out["msda"] = sds.msda_forward(t["v"], shapes, t["loc"], t["attn"])
        out["msda_bwd"] = sds.msda_backward(t["v"], shapes, t["loc"], t["attn"], t["mg"])
        return out

    say("streams: default")
    ref = run(base)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("streams: side")
    with torch.cuda.stream(side):
        for _ in range(3):   # repeat: a race would show on some pass
            t = {k: v.clone() for k, v in base.items()}
            got = run(t)
            side.synchronize()
            assert torch.equal(got["fwd"], ref["fwd"])
            assert torch.equal(got["om"][0], ref["om"][0]) and torch.equal(got["om"][1], ref["om"][1])
            assert torch.equal(got["msda"], ref["msda"])
            for a, b in zip(got["bwd"], ref["bwd"]):
                assert rel_err(to_host(a), to_host(b)) <= TOL["f16"]
            for a, b in zip(got["msda_bwd"], ref["msda_bwd"]):
                assert rel_err(to_host(a), to_host(b)) <= 1e-5


def test_msda_backward_ws_reused_workspace(sds):
    """One caller-owned workspace serves two msda_backward_ws calls in a row,
    the second on a smaller problem: counts and records left by the first
    must not leak into the second.  Both match the oracle at the gather
    path's bars."""
    import ctypes
    import torch
    from sparse_deformable_sampling_amd import _binding as B
    L = B.lib()
    cases = [(2, [(9, 11), (5, 6), (3, 3), (2, 2)], 300, 4, 32, 4, 81), (1, [(6, 7), (3, 4)], 90, 2, 16, 2, 82)]
    sizes = []
    for n, shapes, q, heads, dh, pts, _ in cases:
        desc = B.MsdaDesc(n, q, heads, dh, len(shapes), pts, 1, B.DCN_F32)
        shp = (ctypes.c_int32 * (2 * len(shapes)))(*[v for hw in shapes for v in hw])
        nb = ctypes.c_size_t(0)
        assert L.msda_backward_workspace_size(ctypes.byref(desc), shp, ctypes.byref(nb)) == B.DCN_OK
        sizes.append(nb.value)
    assert sizes[0] > sizes[1] > 0
    ws = torch.empty((sizes[0],), dtype=torch.uint8, device="cuda")
    for n, shapes, q, heads, dh, pts, seed in cases:
        d = synth.msda_inputs(n, shapes, q, heads, dh, pts, seed=seed)
        g = np.random.default_rng(seed).standard_normal((n, q, heads, dh)).astype(np.float32)
        v, lc, at, go = (to_dev(a, "f32") for a in (d["value"], d["loc"], d["attn"], g))
        desc = B.MsdaDesc(n, q, heads, dh, len(shapes), pts, 1, B.DCN_F32)
        shp = (ctypes.c_int32 * (2 * len(shapes)))(*[x for hw in shapes for x in hw])
        out = [torch.empty_like(v), torch.empty_like(lc), torch.empty_like(at)]
        say("msda-bwd-ws-reuse", (n, shapes, q, heads, dh, pts))
        st = L.msda_backward_ws(ctypes.byref(desc), shp, *(ctypes.c_void_p(t.data_ptr()) for t in (v, lc, at, go)),
                                *(ctypes.c_void_p(t.data_ptr()) for t in out), ctypes.c_void_p(ws.data_ptr()),
                                ctypes.c_size_t(sizes[0]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == B.DCN_OK
        torch.cuda.synchronize()
        ref = oracle.msda_backward(d["value"], shapes, d["loc"], d["attn"], g, softmax=True)
        for a, b, tol in zip(out, ref, MSDA_BWD_TOL_GATHER):
            assert rel_err(to_host(a), b) <= tol


# ---------------------------------------------------------------- very wide rows


@pytest.mark.parametrize("w", [1200, 3000])
def test_very_wide_rows(sds, w):
    """Rows thousands of pixels wide: the forward's LDS ring then holds fewer
    groups (or no window at all, and the direct gather runs), the backward's
    fixed-point window fewer rows, and the front-end's sliding window walks
    a long row.  Forward f32/f16/bf16 with both modulations, backward f32 and
    f16, front-end f16/bf16, all against the oracle."""
    n, h, c, g = 1, 6, 64, 4
    for dtype in ("f32", "f16", "bf16"):
        for softmax in (False, True):
            check_fwd(sds, "very-wide", n, h, w, c, g, dtype, softmax, seed=91)
    for dtype in ("f32", "f16"):
        check_bwd(sds, "bwd-very-wide", n, h, w, c, g, False, seed=92, dtype=dtype)
    for dtype in ("f16", "bf16"):
        check_frontend(sds, "frontend-very-wide", n, h, w, c, g, dtype, seed=93)
