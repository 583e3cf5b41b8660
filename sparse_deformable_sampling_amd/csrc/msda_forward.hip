// Multi-scale deformable attention sampling core for gfx950 (fp32).
//
// "Deformable DETR: Learn Where to Read":
//  - "A learned location can fall between cells": a normalised location
//    (u, v) of level l maps to pixel coordinates x = u*W_l - 1/2,
//    y = v*H_l - 1/2; the read is the tent-weighted sum of the four
//    neighbouring cells, a cell outside the level reads zero, and nothing is
//    clamped or renormalised.
//  - "Mix samples with a per-head budget": per query and head, one softmax
//    over all levels and points jointly; the head output is the weighted sum
//    of the sampled head-dim vectors.
//
// Work item = one (image, query, head); a lane holds 4 consecutive channels
// of the head (16-byte loads of the [n][S][heads][head_dim] value tensor) or,
// for other head sizes, the whole head.  The pixel coordinate is formed in
// fp64, where u*W_l - 1/2 and its fraction are exact for any f32 u, so the
// interpolation weights carry only the final rounding to fp32.
#include <algorithm>

#include "dcn_device.h"

namespace dcn {

namespace {

struct Sample {
    float w00, w01, w10, w11;
    long base;   // element index of cell (y0, x0), head h, channel 0, of image n
    bool c00, c01, c10, c11;
    bool any;
};

__device__ __forceinline__ Sample sample_geometry(const MsdaGeom& G, int l, float u, float v, float A, long img_head)
{
    Sample s;
    s.any = false;
    const int Hl = G.H[l], Wl = G.W[l];
    const double x = (double)u * Wl - 0.5, y = (double)v * Hl - 0.5;
    if (!(x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl)) return s;
    const double fx = floor(x), fy = floor(y);
    const float a = (float)(x - fx), b = (float)(y - fy);
    const int x0 = (int)fx, y0 = (int)fy;
    s.c00 = y0 >= 0 && x0 >= 0;
    s.c01 = y0 >= 0 && x0 + 1 < Wl;
    s.c10 = y0 + 1 < Hl && x0 >= 0;
    s.c11 = y0 + 1 < Hl && x0 + 1 < Wl;
    const float Aa = A * (1.f - a), Ab = A * a;
    s.w00 = Aa * (1.f - b);
    s.w01 = Ab * (1.f - b);
    s.w10 = Aa * b;
    s.w11 = Ab * b;
    s.base = img_head + ((long)G.start[l] + (long)y0 * Wl + x0) * G.m * G.dh;
    s.any = true;
    return s;
}

// Joint softmax statistics of one head's L*P logits.
__device__ __forceinline__ void head_stats(const float* a, int LP, bool softmax, float& mx, float& inv)
{
    mx = 0.f;
    inv = 1.f;
    if (!softmax) return;
    mx = a[0];
    for (int i = 1; i < LP; ++i) mx = fmaxf(mx, a[i]);
    float s = 0.f;
    for (int i = 0; i < LP; ++i) s += exp_nonpos(a[i] - mx);
    inv = 1.0f / s;
}

// One lane per (image, query, head, 4 channels); P = head_dim / 4 lanes per item.
template <bool SOFTMAX>
__global__ __launch_bounds__(256) void msda_fwd_vec4(MsdaGeom G, const float* __restrict__ value,
                                                     const float* __restrict__ loc,
                                                     const float* __restrict__ attn, float* __restrict__ out)
{
    const int P4 = G.dh / 4;
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long items = (long)G.n * G.q * G.m;
    const long item = t / P4;
    if (item >= items) return;
    const int chunk = (int)(t - item * P4);
    const int h = (int)(item % G.m);
    const int n = (int)(item / ((long)G.q * G.m));
    const int LP = G.L * G.P;
    const float* ai = attn + item * LP;
    const float* li = loc + item * LP * 2;
    float mx, inv;
    head_stats(ai, LP, SOFTMAX, mx, inv);
    const long img_head = (long)n * G.S * G.m * G.dh + (long)h * G.dh + chunk * 4;
    const long rowstride_unit = (long)G.m * G.dh;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int l = 0; l < G.L; ++l) {
        const long rowc = (long)G.W[l] * rowstride_unit;
        for (int p = 0; p < G.P; ++p) {
            const int i = l * G.P + p;
            const float A = SOFTMAX ? exp_nonpos(ai[i] - mx) * inv : ai[i];
            const Sample s = sample_geometry(G, l, li[2 * i], li[2 * i + 1], A, img_head);
            if (!s.any) continue;
            float v[4];
            if (s.c00) {
                load_vec<DT_F32>(value + s.base, v);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(s.w00, v[c], acc[c]);
            }
            if (s.c01) {
                load_vec<DT_F32>(value + s.base + rowstride_unit, v);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(s.w01, v[c], acc[c]);
            }
            if (s.c10) {
                load_vec<DT_F32>(value + s.base + rowc, v);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(s.w10, v[c], acc[c]);
            }
            if (s.c11) {
                load_vec<DT_F32>(value + s.base + rowc + rowstride_unit, v);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(s.w11, v[c], acc[c]);
            }
        }
    }
    store_vec<DT_F32>(out + item * G.dh + chunk * 4, acc);
}

// Tiled kernel: a workgroup takes QT queries of one (image, head) pair.
//  - Work order: pair-major, and the workgroup IDs are remapped so that each
//    XCD sweeps a contiguous range of pairs (workgroups are handed to the
//    eight XCDs round-robin).  One head's values are S rows of head_dim
//    floats (2.3 MB for the Deformable DETR encoder), which stay in that
//    XCD's L2 while its CUs work through the pair; interleaving all heads
//    would spread the reads over the image's whole value tensor.
//  - Phase 1: one thread per sample computes the joint softmax (shuffles
//    over the LP lanes of a query), the fp64 pixel coordinate and the four
//    corners' byte offsets and weights, into an LDS record.
//  - Phase 2: lane = (query, 4 channels); for every sample it reads the
//    record (a broadcast) and the four 16-byte corner chunks with buffer
//    loads, where a corner outside the level carries an offset past the end
//    of the buffer and reads zero.
constexpr uint32_t MS_OOB = 0x80000000u;
constexpr int MS_REC_MAX = 1024;   // sample records per workgroup (32 KB)

template <bool SOFTMAX>
__global__ __launch_bounds__(256) void msda_fwd_tile(MsdaGeom G, int LPlog, int LQlog, int QT, int tiles, int nwg,
                                                     uint32_t value_bytes, const float* __restrict__ value,
                                                     const float* __restrict__ loc, const float* __restrict__ attn,
                                                     float* __restrict__ out)
{
    __shared__ u32x4 rec_o[MS_REC_MAX];
    __shared__ float4 rec_w[MS_REC_MAX];
    const int nwg_pad = (nwg + 7) & ~7;
    const int b = blockIdx.x;
    const int L = (b & 7) * (nwg_pad >> 3) + (b >> 3);
    if (L >= nwg) return;
    const int pair = L / tiles, tile = L - pair * tiles;
    const int n = pair / G.m, h = pair - n * G.m;
    const int LP = 1 << LPlog;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int q0 = tile * QT;
    const uint32_t unit = (uint32_t)G.m * G.dh * 4u;   // bytes from one value row to the next

    // ---- phase 1: sample records
    const int nsamp = QT << LPlog;
    for (int s = tid; s < nsamp; s += nthr) {
        const int qi = s >> LPlog, i = s & (LP - 1);
        const int q = q0 + qi;
        const bool valid = q < G.q;
        const long item = ((long)n * G.q + (valid ? q : 0)) * G.m + h;
        const float2 uv = *reinterpret_cast<const float2*>(loc + (item * LP + i) * 2);
        float A = attn[item * LP + i];
        if constexpr (SOFTMAX) {
            float mx = A;
            for (int o = 1; o < LP; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float e = exp_nonpos(A - mx);
            float sum = e;
            for (int o = 1; o < LP; o <<= 1) sum += __shfl_xor(sum, o, 64);
            A = e * (1.0f / sum);
        }
        const int l = i / G.P;
        const int Hl = G.H[l], Wl = G.W[l];
        u32x4 o = {MS_OOB, MS_OOB, MS_OOB, MS_OOB};
        float4 w = {0.f, 0.f, 0.f, 0.f};
        const double x = (double)uv.x * Wl - 0.5, y = (double)uv.y * Hl - 0.5;
        if (valid && x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl) {
            const double fx = floor(x), fy = floor(y);
            const float a = (float)(x - fx), bb = (float)(y - fy);
            const int x0 = (int)fx, y0 = (int)fy;
            const float Aa = A * (1.f - a), Ab = A * a;
            w = make_float4(Aa * (1.f - bb), Ab * (1.f - bb), Aa * bb, Ab * bb);
            // byte offset of cell (y0, x0) of this image and head; the value
            // tensor is below 2 GB, and cells outside the level are never used
            const long row = (long)n * G.S + G.start[l] + (long)y0 * Wl + x0;
            const uint32_t base = (uint32_t)(row * G.m + h) * (uint32_t)(G.dh * 4);
            const uint32_t down = (uint32_t)Wl * unit;
            const bool cx0 = x0 >= 0, cx1 = x0 + 1 < Wl, cy0 = y0 >= 0, cy1 = y0 + 1 < Hl;
            o.x = (cy0 && cx0) ? base : MS_OOB;
            o.y = (cy0 && cx1) ? base + unit : MS_OOB;
            o.z = (cy1 && cx0) ? base + down : MS_OOB;
            o.w = (cy1 && cx1) ? base + down + unit : MS_OOB;
        }
        rec_o[s] = o;
        rec_w[s] = w;
    }
    __syncthreads();

    // ---- phase 2: gather and accumulate
    const int qi = tid >> LQlog, chunk = tid & ((1 << LQlog) - 1);
    const int q = q0 + qi;
    if (qi >= QT || q >= G.q) return;
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)value, (short)0, (int)value_bytes,
                                                                        0x00020000);
    const uint32_t cb = 16u * chunk;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int r0 = qi << LPlog;
#pragma unroll 4
    for (int i = 0; i < LP; ++i) {
        const u32x4 o = rec_o[r0 + i];
        const float4 w = rec_w[r0 + i];
        const u32x4 v00 = __builtin_amdgcn_raw_buffer_load_b128(vr, o.x + cb, 0, 0);
        const u32x4 v01 = __builtin_amdgcn_raw_buffer_load_b128(vr, o.y + cb, 0, 0);
        const u32x4 v10 = __builtin_amdgcn_raw_buffer_load_b128(vr, o.z + cb, 0, 0);
        const u32x4 v11 = __builtin_amdgcn_raw_buffer_load_b128(vr, o.w + cb, 0, 0);
        const uint32_t c00[4] = {v00.x, v00.y, v00.z, v00.w}, c01[4] = {v01.x, v01.y, v01.z, v01.w};
        const uint32_t c10[4] = {v10.x, v10.y, v10.z, v10.w}, c11[4] = {v11.x, v11.y, v11.z, v11.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[c] = fmaf(w.x, __uint_as_float(c00[c]), acc[c]);
            acc[c] = fmaf(w.y, __uint_as_float(c01[c]), acc[c]);
            acc[c] = fmaf(w.z, __uint_as_float(c10[c]), acc[c]);
            acc[c] = fmaf(w.w, __uint_as_float(c11[c]), acc[c]);
        }
    }
    const long item = ((long)n * G.q + q) * G.m + h;
    store_vec<DT_F32>(out + item * G.dh + cb / 4, acc);
}

// Any head_dim: one lane per (image, query, head), channel loop.
template <bool SOFTMAX>
__global__ __launch_bounds__(256) void msda_fwd_generic(MsdaGeom G, const float* __restrict__ value,
                                                        const float* __restrict__ loc,
                                                        const float* __restrict__ attn, float* __restrict__ out)
{
    const long item = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long items = (long)G.n * G.q * G.m;
    if (item >= items) return;
    const int h = (int)(item % G.m);
    const int n = (int)(item / ((long)G.q * G.m));
    const int LP = G.L * G.P;
    const float* ai = attn + item * LP;
    const float* li = loc + item * LP * 2;
    float mx, inv;
    head_stats(ai, LP, SOFTMAX, mx, inv);
    const long img_head = (long)n * G.S * G.m * G.dh + (long)h * G.dh;
    const long unit = (long)G.m * G.dh;
    float* o = out + item * G.dh;
    for (int c = 0; c < G.dh; ++c) o[c] = 0.f;
    for (int l = 0; l < G.L; ++l) {
        const long rowc = (long)G.W[l] * unit;
        for (int p = 0; p < G.P; ++p) {
            const int i = l * G.P + p;
            const float A = SOFTMAX ? exp_nonpos(ai[i] - mx) * inv : ai[i];
            const Sample s = sample_geometry(G, l, li[2 * i], li[2 * i + 1], A, img_head);
            if (!s.any) continue;
            for (int c = 0; c < G.dh; ++c) {
                float acc = o[c];
                if (s.c00) acc = fmaf(s.w00, value[s.base + c], acc);
                if (s.c01) acc = fmaf(s.w01, value[s.base + unit + c], acc);
                if (s.c10) acc = fmaf(s.w10, value[s.base + rowc + c], acc);
                if (s.c11) acc = fmaf(s.w11, value[s.base + rowc + unit + c], acc);
                o[c] = acc;
            }
        }
    }
}

}  // namespace

hipError_t launch_msda_forward(const MsdaGeom& G, const float* value, const float* loc, const float* attn, float* out,
                               hipStream_t s)
{
    const long items = (long)G.n * G.q * G.m;
    const bool aligned = ((uintptr_t)value % 16 == 0) && ((uintptr_t)out % 16 == 0) && ((uintptr_t)loc % 8 == 0);
    const dim3 block(256);
    const int LP = G.L * G.P, LQ = G.dh / 4;
    const long value_bytes = (long)G.n * G.S * G.m * G.dh * 4;
    const bool pow2 = (LP & (LP - 1)) == 0 && LP <= 32 && G.dh % 4 == 0 && (LQ & (LQ - 1)) == 0 && LQ <= 64;
    if (aligned && pow2 && value_bytes < (1L << 31) - 64) {
        int LPlog = 0, LQlog = 0;
        while ((1 << LPlog) < LP) ++LPlog;
        while ((1 << LQlog) < LQ) ++LQlog;
        const int QT = std::min(256 / LQ, MS_REC_MAX / LP);
        const int tiles = (G.q + QT - 1) / QT;
        const long nwg = (long)G.n * G.m * tiles;
        if (nwg < (1L << 30)) {
            const dim3 grid((unsigned)((nwg + 7) & ~7L)), blk((unsigned)(QT * LQ));
            if (G.softmax)
                msda_fwd_tile<true><<<grid, blk, 0, s>>>(G, LPlog, LQlog, QT, tiles, (int)nwg, (uint32_t)value_bytes,
                                                         value, loc, attn, out);
            else
                msda_fwd_tile<false><<<grid, blk, 0, s>>>(G, LPlog, LQlog, QT, tiles, (int)nwg, (uint32_t)value_bytes,
                                                          value, loc, attn, out);
            return hipGetLastError();
        }
    }
    if (aligned && G.dh % 4 == 0) {
        const long lanes = items * (G.dh / 4);
        const dim3 grid((unsigned)((lanes + 255) / 256));
        if (G.softmax) msda_fwd_vec4<true><<<grid, block, 0, s>>>(G, value, loc, attn, out);
        else msda_fwd_vec4<false><<<grid, block, 0, s>>>(G, value, loc, attn, out);
    } else {
        const dim3 grid((unsigned)((items + 255) / 256));
        if (G.softmax) msda_fwd_generic<true><<<grid, block, 0, s>>>(G, value, loc, attn, out);
        else msda_fwd_generic<false><<<grid, block, 0, s>>>(G, value, loc, attn, out);
    }
    return hipGetLastError();
}

}  // namespace dcn
