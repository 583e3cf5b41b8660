#!/usr/bin/env python3
"""Benchmark of libdcn on one MI355X.

Headline: DCNv4 forward (no softmax, mask N(0,1) unbounded) at the
InternImage-T stage-1 shape N=64, H=W=56, C=64, G=4 (16 channels per group),
3x3 kernel, stride 1, pad 1, in f16 with fp32 accumulation; offsets N(0,1.5).
A step is one dcn_forward call over the batch.  Inputs are resident in HBM
before the timed region and rotate over enough copies (>= 1 GB in all) that
no step finds its inputs in the 256 MB Infinity Cache or the L2s.

Printed: ONE JSON line with the throughput in Gtaps*ch/s (N*Ho*Wo*C*K per
second), the roofline of the kernel against the minimum-traffic model
(x read once + offsets + mask + output written once), the CPU oracle's own
throughput on this host, and secondary figures for the other entry points.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DCN fwd Gtaps*ch/s and achieved HBM GB/s (% of peak), InternImage-T stage-1 shape"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30
ES = {"f32": 4, "f16": 2, "bf16": 2}

STAGES = {"stage1": (64, 56, 56, 64, 4), "stage2": (64, 28, 28, 128, 8), "stage3": (64, 14, 14, 320, 20),
          # the DCNv4 pages' module measurement: 56x56x128, batch 64, 4 groups of 32 channels
          "table10": (64, 56, 56, 128, 4)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None, help="run only this workload (profiling)")
    return ap.parse_args()


class Runner:
    """A prepared sequence of launches over rotating copies of one input set."""

    def __init__(self, name, launch_args, fn, units, min_bytes, stream):
        self.name, self.args, self.fn, self.units, self.min_bytes, self.stream = (
            name, launch_args, fn, units, min_bytes, stream)

    def launch(self, i):
        st = self.fn(*self.args[i % len(self.args)])
        if st != 0:
            from sparse_deformable_sampling_amd import _binding as B
            raise B.DcnError(st)


def upload(torch, a, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to("cuda")


def n_sets(bytes_per_set):
    return max(2, int(math.ceil(ROTATE_BYTES / bytes_per_set)))


def dcn_fwd_runner(torch, stage, dtype, softmax, seed=1):
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, h, w, c, g = STAGES[stage]
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype=dtype, seed=seed)
    es = ES[dtype]
    elems = d["x"].size + d["offset"].size + d["mask"].size + n * h * w * c
    min_bytes = elems * es
    code = {"f32": B.DCN_F32, "f16": B.DCN_F16, "bf16": B.DCN_BF16}[dtype]
    desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, softmax, code)
    base = [upload(torch, d[k], dtype) for k in ("x", "offset", "mask")]
    stream = torch.cuda.current_stream()
    args, keep = [], []
    for i in range(n_sets(min_bytes)):
        x, off, mask = (t.clone() for t in base) if i else base
        out = torch.empty((n, h, w, c), dtype=x.dtype, device="cuda")
        keep += [x, off, mask, out]
        args.append((ctypes.byref(desc), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(off.data_ptr()),
                     ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                     ctypes.c_void_p(stream.cuda_stream)))
    r = Runner("%s_fwd_%s_%s" % ("dcnv3" if softmax else "dcnv4", stage, dtype), args, B.lib().dcn_forward,
               n * h * w * c * 9, min_bytes, stream)
    r.keep, r.desc, r.inputs = keep, desc, d
    return r


def dcn_bwd_runner(torch, softmax, seed=1, stage="stage1", dtype="f32"):
    """DCN backward through dcn_backward_ws (an fp32 grad_x workspace for
    f16/bf16, none for f32).  min_bytes counts the tensors the op reads (x,
    offset, mask, grad_out) and writes (grad_x, grad_offset, grad_mask) once,
    in their own dtype; the workspace's fp32 traffic is not algorithmic."""
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, h, w, c, g = STAGES[stage]
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype=dtype, seed=seed, grad=True)
    es = ES[dtype]
    elems = 2 * (d["x"].size + d["offset"].size + d["mask"].size) + d["grad_out"].size
    min_bytes = elems * es
    code = {"f32": B.DCN_F32, "f16": B.DCN_F16, "bf16": B.DCN_BF16}[dtype]
    desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, softmax, code)
    nbytes = ctypes.c_size_t(0)
    B.check(B.lib().dcn_backward_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)))
    base = [upload(torch, d[k], dtype) for k in ("x", "offset", "mask", "grad_out")]
    stream = torch.cuda.current_stream()
    args, keep = [], []
    for i in range(n_sets(min_bytes)):
        ins = [t.clone() for t in base] if i else base
        outs = [torch.empty_like(ins[0]), torch.empty_like(ins[1]), torch.empty_like(ins[2])]
        ws = torch.empty(((nbytes.value + 3) // 4,), dtype=torch.float32, device="cuda") if nbytes.value else None
        keep += ins + outs + [ws]
        args.append((ctypes.byref(desc),) + tuple(ctypes.c_void_p(t.data_ptr()) for t in ins + outs) +
                    (ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), ctypes.c_size_t(nbytes.value),
                     ctypes.c_void_p(stream.cuda_stream)))
    r = Runner("%s_bwd_%s_%s" % ("dcnv3" if softmax else "dcnv4", stage, dtype), args, B.lib().dcn_backward_ws,
               n * h * w * c * 9, min_bytes, stream)
    r.keep = keep
    return r


FRONT_KEYS = ("x", "dw_weight", "dw_bias", "om_weight", "om_bias")


def frontend_runner(torch, stage, dtype, seed=1):
    """DCNv4 front-end (dcn_offset_mask): min_bytes counts x, the weights and
    the offset and mask outputs once."""
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, h, w, c, g = STAGES[stage]
    d = synth.frontend_inputs(n, h, w, c, g, dtype=dtype, seed=seed)
    es = ES[dtype]
    min_bytes = es * (sum(d[k].size for k in FRONT_KEYS) + n * h * w * g * 27)
    code = {"f16": B.DCN_F16, "bf16": B.DCN_BF16}[dtype]
    desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, False, code)
    base = [upload(torch, d[k], dtype) for k in FRONT_KEYS]
    stream = torch.cuda.current_stream()
    args, keep = [], []
    for i in range(n_sets(min_bytes)):
        ins = [base[0].clone()] + base[1:] if i else base
        off = torch.empty((n, h, w, g, 9, 2), dtype=ins[0].dtype, device="cuda")
        mask = torch.empty((n, h, w, g, 9), dtype=ins[0].dtype, device="cuda")
        keep += ins + [off, mask]
        args.append((ctypes.byref(desc),) + tuple(ctypes.c_void_p(t.data_ptr()) for t in ins + [off, mask]) +
                    (ctypes.c_void_p(stream.cuda_stream),))
    r = Runner("dcnv4_offset_mask_%s_%s" % (stage, dtype), args, B.lib().dcn_offset_mask, n * h * w * c * 9,
               min_bytes, stream)
    r.keep = keep
    return r


def module_runner(torch, stage="table10", dtype="f16", seed=1):
    """The whole DCNv4 module forward, as the pages measure it (Table 10):
    value = input_proj(x) and out = output_proj(core(...)) as plain library
    GEMMs (torch.mm on the same stream), the front-end and the core in
    libdcn (dcn_offset_mask, then dcn_forward).  min_bytes sums each step's
    own reads and writes once, x read once: 6*P*C elements for P pixels,
    plus 2*P*G*K*3 for the offsets and mask written and read between the
    two launches (weights aside)."""
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, h, w, c, g = STAGES[stage]
    d = synth.frontend_inputs(n, h, w, c, g, dtype=dtype, seed=seed)
    es = ES[dtype]
    P = n * h * w
    min_bytes = es * (6 * P * c + 2 * P * g * 27)
    code = {"f16": B.DCN_F16, "bf16": B.DCN_BF16}[dtype]
    desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, False, code)
    fe = [upload(torch, d[k], dtype) for k in FRONT_KEYS]
    rng = np.random.default_rng(seed + 77)
    w_in, w_out = (upload(torch, synth.store((rng.standard_normal((c, c)) / math.sqrt(c)).astype(np.float32), dtype), dtype)
                   for _ in range(2))   # [in][out]: x @ w
    stream = torch.cuda.current_stream()
    L = B.lib()
    sets = []
    for i in range(n_sets(min_bytes)):
        x = fe[0].clone() if i else fe[0]
        t = dict(x=x, value=torch.empty((P, c), dtype=x.dtype, device="cuda"),
                 off=torch.empty((n, h, w, g, 9, 2), dtype=x.dtype, device="cuda"),
                 mask=torch.empty((n, h, w, g, 9), dtype=x.dtype, device="cuda"),
                 y=torch.empty((P, c), dtype=x.dtype, device="cuda"), out=torch.empty((P, c), dtype=x.dtype, device="cuda"))
        sets.append(t)
    vp = ctypes.c_void_p
    sp = vp(stream.cuda_stream)

    def step(t):
        torch.mm(t["x"].view(P, c), w_in, out=t["value"])
        st = L.dcn_offset_mask(ctypes.byref(desc), vp(t["x"].data_ptr()), *(vp(a.data_ptr()) for a in fe[1:]),
                               vp(t["off"].data_ptr()), vp(t["mask"].data_ptr()), sp)
        if st == 0:
            st = L.dcn_forward(ctypes.byref(desc), vp(t["value"].data_ptr()), vp(t["off"].data_ptr()),
                               vp(t["mask"].data_ptr()), vp(t["y"].data_ptr()), sp)
        torch.mm(t["y"], w_out, out=t["out"])
        return st

    r = Runner("dcnv4_module_%s_%s" % (stage, dtype), [(t,) for t in sets], step, n * h * w * c * 9, min_bytes,
               stream)
    r.keep = (fe, w_in, w_out, sets)
    return r


MSDA_SHAPES = [(100, 134), (50, 67), (25, 34), (13, 17)]


def msda_runner(torch, seed=1):
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, q, heads, dh, pts = 8, 17821, 8, 32, 4
    d = synth.msda_inputs(n, MSDA_SHAPES, q, heads, dh, pts, seed=seed, ref="cells")
    min_bytes = 4 * (d["value"].size + d["loc"].size + d["attn"].size + n * q * heads * dh)
    desc = B.MsdaDesc(n, q, heads, dh, len(MSDA_SHAPES), pts, 1, B.DCN_F32)
    shapes = (ctypes.c_int32 * 8)(*[v for hw in MSDA_SHAPES for v in hw])
    base = [upload(torch, d[k], "f32") for k in ("value", "loc", "attn")]
    stream = torch.cuda.current_stream()
    args, keep = [], []
    for i in range(n_sets(min_bytes)):
        ins = [t.clone() for t in base] if i else base
        out = torch.empty((n, q, heads, dh), device="cuda")
        keep += ins + [out]
        args.append((ctypes.byref(desc), shapes) + tuple(ctypes.c_void_p(t.data_ptr()) for t in ins + [out]) +
                    (ctypes.c_void_p(stream.cuda_stream),))
    r = Runner("msda_fwd_encoder_f32", args, B.lib().msda_forward, n * q * heads * dh * len(MSDA_SHAPES) * pts,
               min_bytes, stream)
    r.keep = keep
    return r


# The MSDA gather's second ceiling: every corner read of a head is one
# 128-byte line (32 fp32 channels, line-aligned), and the vector L1 looks up
# about 0.43 lines per clock per CU (measured on gfx950 with scattered 16-byte
# reads), so 4 lines per sample bound the kernel below the HBM roofline.
L1_LINES_PER_CLK_CU = 0.43
CU_COUNT, CLOCK_GHZ = 256, 2.4


def msda_line_roofline(kernel_us):
    n, q, heads, pts = 8, 17821, 8, 4
    lines = n * q * heads * len(MSDA_SHAPES) * pts * 4
    floor_us = lines / (L1_LINES_PER_CLK_CU * CU_COUNT * CLOCK_GHZ * 1e3)
    return {"bound": "vector L1 line lookups", "lines_per_launch": lines, "lines_per_clk_per_cu": L1_LINES_PER_CLK_CU,
            "floor_us": round(floor_us, 1), "frac": round(floor_us / kernel_us, 4)}


# fp32 multiply-add issue rate without packed fp32 instructions (which this
# library does not use): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
VALU_FMA_PEAK_TFLOPS = CU_COUNT * 4 * 16 * 2 * CLOCK_GHZ / 1e3


def valu_roofline(kernel_us, items=64 * 56 * 56 * 4, d=16, taps=9):
    """The headline's second ceiling, the vector ALU: its arithmetic is one
    fp32 multiply-add per (item, channel, tap, corner), 2 flops each (the
    tap geometry, computed once per item and tap, comes on top)."""
    flops = items * d * taps * 4 * 2
    achieved = flops / (kernel_us * 1e-6) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 2), "peak": round(VALU_FMA_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FMA_PEAK_TFLOPS, 4), "flops_per_launch": flops,
            "flops": "4 corners x 9 taps x D channels x 2 per (pixel, group) item: the bilinear multiply-adds in fp32"}


def msda_ref_runner(torch, seed=1):
    """MSDA read with locations formed in the kernel: the encoder shape with
    per-image valid ratios and right/bottom padding, every cell a query that
    refers to its own cell centre in the valid frame (the encoder's
    reference points, as msda_runner's locations).  min_bytes: value,
    offsets, attn and out once, plus the references, ratios and the byte
    mask."""
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, q, heads, dh, pts = 8, 17821, 8, 32, 4
    d = synth.msda_ref_inputs(n, MSDA_SHAPES, q, heads, dh, pts, ref_dims=2, padded=True, seed=seed, ref="cells")
    min_bytes = 4 * (d["value"].size + d["offsets"].size + d["attn"].size + n * q * heads * dh +
                     d["reference"].size + d["valid_ratios"].size) + d["padding_mask"].size
    desc = B.MsdaDesc(n, q, heads, dh, len(MSDA_SHAPES), pts, 1, B.DCN_F32)
    shapes = (ctypes.c_int32 * 8)(*[v for hw in MSDA_SHAPES for v in hw])
    base = [upload(torch, d[k], "f32") for k in ("value", "reference", "valid_ratios", "offsets", "attn")]
    base.append(torch.from_numpy(d["padding_mask"]).cuda())
    stream = torch.cuda.current_stream()
    args, keep = [], []
    for i in range(n_sets(min_bytes)):
        ins = [t.clone() for t in base] if i else base
        out = torch.empty((n, q, heads, dh), device="cuda")
        keep += ins + [out]
        v, ref, rat, off, att, pad = (ctypes.c_void_p(t.data_ptr()) for t in ins)
        args.append((ctypes.byref(desc), shapes, ctypes.c_int32(2), v, ref, rat, off, att, pad,
                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)))
    r = Runner("msda_fwd_ref_encoder_f32", args, B.lib().msda_forward_ref, n * q * heads * dh * len(MSDA_SHAPES) * pts,
               min_bytes, stream)
    r.keep = keep
    return r


def msda_bwd_runner(torch, gather=True, seed=1):
    """gather=True: grad_value gathered per cell through one workspace shared by
    all launches (they run in order on one stream); False: atomic scatter."""
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, q, heads, dh, pts = 8, 17821, 8, 32, 4
    d = synth.msda_inputs(n, MSDA_SHAPES, q, heads, dh, pts, seed=seed, ref="cells")
    g = np.random.default_rng(seed + 1000).standard_normal((n, q, heads, dh)).astype(np.float32)
    # value, loc, attn, grad_out read; grad_value, grad_loc, grad_attn written once
    min_bytes = 4 * (2 * (d["value"].size + d["loc"].size + d["attn"].size) + g.size)
    desc = B.MsdaDesc(n, q, heads, dh, len(MSDA_SHAPES), pts, 1, B.DCN_F32)
    shapes = (ctypes.c_int32 * 8)(*[v for hw in MSDA_SHAPES for v in hw])
    base = [upload(torch, a, "f32") for a in (d["value"], d["loc"], d["attn"], g)]
    stream = torch.cuda.current_stream()
    args, keep = [], []
    ws_args = ()
    if gather:
        nb = ctypes.c_size_t(0)
        B.check(B.lib().msda_backward_workspace_size(ctypes.byref(desc), shapes, ctypes.byref(nb)))
        ws = torch.empty((nb.value,), dtype=torch.uint8, device="cuda")
        keep.append(ws)
        ws_args = (ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nb.value))
    for i in range(n_sets(min_bytes)):
        ins = [t.clone() for t in base] if i else base
        outs = [torch.empty_like(ins[0]), torch.empty_like(ins[1]), torch.empty_like(ins[2])]
        keep += ins + outs
        args.append((ctypes.byref(desc), shapes) + tuple(ctypes.c_void_p(t.data_ptr()) for t in ins + outs) +
                    ws_args + (ctypes.c_void_p(stream.cuda_stream),))
    r = Runner("msda_bwd_encoder_f32" if gather else "msda_bwd_atomic_encoder_f32", args,
               B.lib().msda_backward_ws if gather else B.lib().msda_backward,
               n * q * heads * dh * len(MSDA_SHAPES) * pts, min_bytes, stream)
    r.keep = keep
    return r


def time_steps(torch, r, steps, warmup):
    """Contract timing: warmup, then exactly `steps` launches bracketed by
    synchronisation.  One HIP event pair, recorded on the launch stream
    around the same `steps` launches, gives the kernel's average launch
    duration over the timed region, so the roofline describes the run the
    headline rate comes from (and kernel time <= step time).
    Returns (wall ms per step, event ms per launch)."""
    for i in range(warmup):
        r.launch(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(r.stream)
    for i in range(steps):
        r.launch(warmup + i)
    b.record(r.stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, a.elapsed_time(b) / steps


def launch_spread(torch, r, steps):
    """Median, p10 and p90 of single launches, each between its own event
    pair on the launch stream (a separate pass after the timed region; each
    figure also carries the event and dispatch latency of one launch)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(r.stream)
        r.launch(i)
        b.record(r.stream)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(d)), float(np.percentile(d, 10)), float(np.percentile(d, 90))


def measure(torch, r, steps, warmup):
    ms_step, mean = time_steps(torch, r, steps, warmup)
    return summarize(r, ms_step, (mean,) + launch_spread(torch, r, steps))


def summarize(r, ms_step, kms):
    mean, med, p10, p90 = kms
    gbs = r.min_bytes / (mean * 1e-3) / 1e9
    return {"ms_per_step": round(ms_step, 5), "kernel_us_mean": round(mean * 1e3, 2),
            "kernel_us_median_single": round(med * 1e3, 2), "kernel_us_p10_single": round(p10 * 1e3, 2),
            "kernel_us_p90_single": round(p90 * 1e3, 2), "min_bytes": int(r.min_bytes),
            "gtaps_ch_per_s": round(r.units / (ms_step * 1e-3) / 1e9, 2),
            "achieved_gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


COPY_CALIB_BYTES = 256 << 20

# Source files that make up the headline kernel; a recorded traffic figure
# is reported only while their hash matches the one recorded with it.
HEADLINE_KERNEL_SOURCES = ["dcn_forward_ring.hip", "dcn_ring.h", "dcn_device.h", "dcn_launch.h"]
HEADLINE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dcn_fwd_ring_f16_stage1_traffic.txt")
HEADLINE_KERNEL = "dcn_fwd_ring (f16, 3x3, DCNv4)"


def kernel_source_hash(files=HEADLINE_KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_deformable_sampling_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_counters():
    """(HBM bytes per launch, L2 hit rate) of the headline kernel from the
    committed counter summary: FETCH_SIZE and WRITE_SIZE, each scaled by what
    the same counter reads for a plain copy of known size, and TCC_HIT /
    (TCC_HIT + TCC_MISS).  Each is None when the summary lacks it or the
    kernel's sources have changed since it was taken."""
    try:
        with open(HEADLINE_TRAFFIC_FILE) as fh:
            fields = dict(l.split(":", 1) for l in fh.read().splitlines() if ":" in l and not l.startswith(" "))
    except OSError:
        return None, None
    if fields.get("kernel_source_sha256", "").strip() != kernel_source_hash():
        return None, None
    out = []
    for key, conv in (("traffic_bytes_per_launch", int), ("l2_hit_rate", float)):
        try:
            out.append(conv(fields[key].strip()))
        except (KeyError, ValueError):
            out.append(None)
    return tuple(out)


def copy_calib(torch, steps, warmup):
    """A plain device-to-device copy of COPY_CALIB_BYTES per launch over
    rotating buffers: the known-size reference that scales the memory-side
    byte counters (FETCH_SIZE, WRITE_SIZE) read for the kernels."""
    nel = COPY_CALIB_BYTES // 4
    bufs = [torch.empty(nel, dtype=torch.float32, device="cuda").fill_(i) for i in range(8)]
    for i in range(warmup + steps):
        bufs[(2 * i + 1) % 8].copy_(bufs[(2 * i) % 8])
    torch.cuda.synchronize()
    print(json.dumps({"only": "copy_calib", "bytes_read": COPY_CALIB_BYTES, "bytes_written": COPY_CALIB_BYTES,
                      "launches": warmup + steps}), flush=True)
    return 0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class pinned_core:
    """Run the calling thread on one host core (the lowest it may use) for
    the duration of a `with` block; the core's number is `.core`."""

    def __enter__(self):
        self.old = os.sched_getaffinity(0)
        self.core = min(self.old)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.old)
        return False


def cpu_baseline(seconds):
    """The CPU oracle as it stands (single-threaded C, double), timed on one
    pinned host core over whole stage-1 DCNv4 f16 batches until `seconds`
    have passed."""
    import oracle
    from sparse_deformable_sampling_amd import synth
    n, h, w, c, g = STAGES["stage1"]
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f16", seed=1)
    oracle.dcn_forward(d["x"][:1], d["offset"][:1], d["mask"][:1], group=g, dtype="f16")  # load/compile
    with pinned_core() as pin:
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.dcn_forward(d["x"], d["offset"], d["mask"], group=g, dtype="f16")
            runs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    units = runs * n * h * w * c * 9
    return {"value": round(units / el / 1e9, 4), "unit": "Gtaps*ch/s", "cores": 1, "kind": "oracle",
            "pinned_core": pin.core, "cpu_model": cpu_model(),
            "sample": "%d full batch(es) of the headline workload (N=64 56x56x64 G=4, DCNv4, f16 inputs read "
                      "as exact doubles) through the single-threaded C oracle on host core %d, %.1f s"
                      % (runs, pin.core, el)}


def tiny_line(torch, reps=200):
    """The tiny DCNv3 f32 case (N=1, 8x8, C=16, G=2, offsets U(-2,2), logits
    N(0,1) with softmax): latency-bound, so the GPU figure is the median of
    single launches between event pairs, and the oracle's the median of 5
    runs on one pinned host core."""
    import oracle
    from sparse_deformable_sampling_amd import _binding as B, synth
    n, h, w, c, g = 1, 8, 8, 16, 2
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), offset=("uniform", -2.0, 2.0), dtype="f32", seed=1)
    desc = B.make_desc(n, h, w, c, g, 3, 1, 1, 1, 1.0, True, B.DCN_F32)
    x, off, mask = (upload(torch, d[k], "f32") for k in ("x", "offset", "mask"))
    out = torch.empty((n, h, w, c), device="cuda")
    stream = torch.cuda.current_stream()
    args = [(ctypes.byref(desc), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(off.data_ptr()),
             ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))]
    r = Runner("dcnv3_fwd_tiny_f32", args, B.lib().dcn_forward, n * h * w * c * 9, 0, stream)
    for i in range(20):
        r.launch(i)
    torch.cuda.synchronize()
    med, p10, p90 = launch_spread(torch, r, reps)
    cpu = []
    with pinned_core() as pin:
        for _ in range(5):
            t0 = time.perf_counter()
            oracle.dcn_forward(d["x"], d["offset"], d["mask"], group=g, softmax=True)
            cpu.append(time.perf_counter() - t0)
    return {"gpu_us_median_single": round(med * 1e3, 2), "gpu_us_p10_single": round(p10 * 1e3, 2),
            "gpu_us_p90_single": round(p90 * 1e3, 2), "single_launches": reps,
            "cpu_oracle_us_median_of_5": round(float(np.median(cpu)) * 1e6, 2), "cpu_pinned_core": pin.core,
            "taps_ch": n * h * w * c * 9}


def cpu_baseline_threads(seconds, max_threads=16):
    """The same unmodified oracle, batch-sharded one image per task over the
    host's cores (a thread pool: the oracle's C call releases the GIL)."""
    import concurrent.futures as cf
    import oracle
    from sparse_deformable_sampling_amd import synth
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, max_threads))
    n, h, w, c, g = STAGES["stage1"]
    d = synth.dcn_inputs(n, h, w, c, g, (h, w), dtype="f16", seed=1)
    one = lambda i: oracle.dcn_forward(d["x"][i:i + 1], d["offset"][i:i + 1], d["mask"][i:i + 1], group=g,
                                       dtype="f16")
    one(0)
    runs, t0 = 0, time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as pool:
        while True:
            list(pool.map(one, range(n)))
            runs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    units = runs * n * h * w * c * 9
    return {"value": round(units / el / 1e9, 4), "unit": "Gtaps*ch/s", "cores": threads, "kind": "oracle",
            "sample": "%d full batch(es) of the headline workload, one image per task on %d threads, %.1f s"
                      % (runs, threads, el)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (the operator would "
              "shard over the batch with no exchange between GPUs)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    from sparse_deformable_sampling_amd import _binding as B
    B.lib()
    if args.only:
        name = args.only
        if name == "copy_calib":
            return copy_calib(torch, args.steps, args.warmup)
        if name.startswith("dcnv4_offset_mask"):
            parts = name.split("_")   # dcnv4_offset_mask_table10_f16
            r = frontend_runner(torch, parts[3], parts[4])
        elif name.startswith("dcnv4_module"):
            parts = name.split("_")   # dcnv4_module_table10_f16
            r = module_runner(torch, parts[2], parts[3])
        elif name.startswith("msda_bwd"):
            r = msda_bwd_runner(torch, gather="atomic" not in name)
        elif name.startswith("msda_fwd_ref"):
            r = msda_ref_runner(torch)
        elif name.startswith("msda"):
            r = msda_runner(torch)
        elif "_bwd_" in name:
            parts = name.split("_")   # dcnv4_bwd_stage1_f32
            r = dcn_bwd_runner(torch, name.startswith("dcnv3"), stage=parts[2], dtype=parts[3])
        else:
            parts = name.split("_")   # dcnv4_fwd_stage1_f16
            r = dcn_fwd_runner(torch, parts[2], parts[3], parts[0] == "dcnv3")
        print(json.dumps({"only": r.name, **measure(torch, r, args.steps, args.warmup)}), flush=True)
        return 0

    head = dcn_fwd_runner(torch, "stage1", "f16", False)
    s = measure(torch, head, args.steps, args.warmup)
    print("[bench] headline %s: %s" % (head.name, s), file=sys.stderr, flush=True)
    del head

    secondary = {}
    if not args.no_secondary:
        jobs = [("dcnv4", "stage1", "f32"), ("dcnv4", "stage1", "bf16"), ("dcnv3", "stage1", "f32"),
                ("dcnv3", "stage1", "f16"), ("dcnv4", "stage2", "f16"), ("dcnv4", "stage2", "bf16"),
                ("dcnv4", "stage3", "f16"), ("dcnv4", "stage3", "bf16"), ("dcnv4", "table10", "f16"),
                ("dcnv4", "table10", "f32")]
        for kind, stage, dt in jobs:
            r = dcn_fwd_runner(torch, stage, dt, kind == "dcnv3")
            secondary[r.name] = measure(torch, r, 100, 10)
            print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
            del r
        bwd_jobs = [(True, "stage1", "f32"), (False, "stage1", "f32"), (False, "stage1", "f16"),
                    (False, "stage1", "bf16"), (False, "stage2", "f16"), (False, "stage3", "f16")]
        for softmax, stage, dt in bwd_jobs:
            r = dcn_bwd_runner(torch, softmax, stage=stage, dtype=dt)
            secondary[r.name] = measure(torch, r, 50, 5)
            print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
            del r
        for stage, dt in (("table10", "f16"), ("table10", "bf16"), ("stage1", "f16"), ("stage2", "f16"),
                          ("stage3", "f16")):
            r = frontend_runner(torch, stage, dt)
            secondary[r.name] = measure(torch, r, 100, 10)
            print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
            del r
        r = module_runner(torch, "table10", "f16")
        secondary[r.name] = measure(torch, r, 50, 5)
        secondary[r.name]["context_pages_a100_fp16_ms"] = 0.873
        print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
        del r
        for runner in (msda_runner, msda_ref_runner):
            r = runner(torch)
            secondary[r.name] = measure(torch, r, 50, 5)
            secondary[r.name]["l1_line_roofline"] = msda_line_roofline(secondary[r.name]["kernel_us_mean"])
            print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
            del r
        for gather in (True, False):
            r = msda_bwd_runner(torch, gather=gather)
            k = 20 if gather else 5
            secondary[r.name] = measure(torch, r, k, 2)
            print("[bench] %s: %s" % (r.name, secondary[r.name]), file=sys.stderr, flush=True)
            del r
        torch.cuda.empty_cache()

    tiny = tiny_line(torch)
    print("[bench] tiny: %s" % tiny, file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)
    traffic, l2_hit = recorded_counters()
    line = {
        "metric": METRIC, "value": s["gtaps_ch_per_s"], "unit": "Gtaps*ch/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": s["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "dcnv4_fwd_stage1_f16", "n": 64, "h": 56, "w": 56, "c": 64, "group": 4,
                   "kernel": [3, 3], "stride": [1, 1], "pad": [1, 1], "dil": [1, 1], "offset_scale": 1.0,
                   "softmax": 0, "accumulate": "f32", "x": "N(0,1)", "offsets": "N(0,1.5)", "mask": "N(0,1)",
                   "rotating_input_sets": n_sets(s["min_bytes"])},
        "roofline": {"bound": "hbm", "achieved": s["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": s["frac_of_hbm_peak"], "traffic": traffic, "l2_hit_rate": l2_hit,
                     "kernel": HEADLINE_KERNEL, "kernel_us_mean": s["kernel_us_mean"],
                     "kernel_us_median_single": s["kernel_us_median_single"],
                     "algorithmic_bytes_per_launch": s["min_bytes"],
                     "algorithmic_bytes": "(2*D + 3*K) * 2 B per (pixel, group) item: x read once, offsets, mask, "
                                          "out written once; 118 B x 802816 items"},
        "roofline_valu": valu_roofline(s["kernel_us_mean"]),
        "tiny_dcnv3_f32": tiny,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": None if args.no_cpu_baseline else cpu_baseline_threads(args.cpu_seconds),
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
