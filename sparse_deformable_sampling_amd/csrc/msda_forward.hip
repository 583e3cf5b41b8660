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
    const bool aligned = ((uintptr_t)value % 16 == 0) && ((uintptr_t)out % 16 == 0);
    const dim3 block(256);
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
