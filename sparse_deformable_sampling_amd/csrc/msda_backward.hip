// Multi-scale deformable attention backward for gfx950 (fp32).
//
// Gradients of the sampling core ("Deformable DETR: Learn Where to Read":
// "A learned location can fall between cells" -- the read is a function of
// the location; "Mix samples with a per-head budget" -- one softmax per query
// and head over all levels and points).  For sample i of a query and head at
// x = u*W_l - 1/2, y = v*H_l - 1/2 with fractions (a, b), corners V_rc (zero
// outside the level), weight A_i and output gradient g:
//   dL/dV_rc  += A_i * (corner weight) * g                       (fp32 atomics)
//   dL/dA_i    = <g, s_i>,  s_i the bilinear read
//   dL/du_i    = W_l A_i <g, (1-b)(V01-V00) + b(V11-V10)>
//   dL/dv_i    = H_l A_i <g, (1-a)(V10-V00) + a(V11-V01)>
//   dL/dz_i    = A_i (dL/dA_i - sum_j A_j dL/dA_j)                (softmax)
//
// Tiled kernel, the same decomposition as the tiled forward: a workgroup
// takes QT queries of one (image, head) pair, with the pairs swept per XCD.
//  - Phase 1, one thread per sample: joint softmax, fp64 pixel coordinate,
//    the four corners' byte offsets (past the end of the buffer for a corner
//    outside the level) and (a, b, A) into LDS.
//  - Phase 2, lane = (query, channel): for every sample, read the four corner
//    values of this channel, scatter A*w*g into grad_value with buffer
//    atomics (the head_dim lanes of a query add to one contiguous run, the
//    access pattern fp32 atomics serve fastest; out-of-range corners are
//    dropped by the buffer range check), and reduce the three channel sums
//    across the query's lanes; the query's first lane writes (dL/du, dL/dv,
//    A, dL/dA) back into the sample's LDS record.
//  - Phase 3, one thread per sample: softmax backward over the query's
//    samples, coalesced stores of grad_loc and grad_attn.
#include <algorithm>

#include "dcn_device.h"

namespace dcn {

namespace {

constexpr uint32_t MS_OOB = 0x80000000u;
constexpr int MS_REC_MAX = 1024;

__device__ __forceinline__ float lane_sum(float v, int width)
{
    for (int o = 1; o < width; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <bool SOFTMAX>
__global__ __launch_bounds__(256) void msda_bwd_tile(MsdaGeom G, int LPlog, int Dlog, int QT, int tiles, int nwg,
                                                     uint32_t value_bytes, const float* __restrict__ value,
                                                     const float* __restrict__ loc, const float* __restrict__ attn,
                                                     const float* __restrict__ gout, float* __restrict__ gvalue,
                                                     float* __restrict__ gloc, float* __restrict__ gattn)
{
    __shared__ u32x4 rec_o[MS_REC_MAX];
    __shared__ float4 rec_f[MS_REC_MAX];
    const int nwg_pad = (nwg + 7) & ~7;
    const int b = blockIdx.x;
    const int L = (b & 7) * (nwg_pad >> 3) + (b >> 3);
    if (L >= nwg) return;
    const int pair = L / tiles, tile = L - pair * tiles;
    const int n = pair / G.m, h = pair - n * G.m;
    const int LP = 1 << LPlog;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int q0 = tile * QT;
    const uint32_t unit = (uint32_t)G.m * G.dh * 4u;
    const int nsamp = QT << LPlog;

    // ---- phase 1: sample records
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
        float fa = 0.f, fb = 0.f;
        const double x = (double)uv.x * Wl - 0.5, y = (double)uv.y * Hl - 0.5;
        if (valid && x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl) {
            const double fx = floor(x), fy = floor(y);
            fa = (float)(x - fx);
            fb = (float)(y - fy);
            const int x0 = (int)fx, y0 = (int)fy;
            // byte offset of cell (y0, x0) of this image and head (modulo 2^32:
            // only the offsets of cells inside the level are used)
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
        rec_f[s] = make_float4(fa, fb, A, 0.f);
    }
    __syncthreads();

    // ---- phase 2: lane = (query, channel)
    {
        const int D = 1 << Dlog;
        const int qi = tid >> Dlog, c = tid & (D - 1);
        const int q = q0 + qi;
        const bool live = qi < QT && q < G.q;
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)value, (short)0, (int)value_bytes,
                                                                            0x00020000);
        const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc((void*)gvalue, (short)0,
                                                                            gvalue ? (int)value_bytes : 0, 0x00020000);
        const long item = ((long)n * G.q + (live ? q : 0)) * G.m + h;
        const float g = live ? gout[item * G.dh + c] : 0.f;
        const uint32_t cb = 4u * c;
        const int r0 = (live ? qi : 0) << LPlog;
        // Lanes of a query that is past the end still take part in the
        // reductions (with g = 0) and write nothing.
        for (int i = 0; i < LP; ++i) {
            const u32x4 o = rec_o[r0 + i];
            const float4 f = rec_f[r0 + i];
            const float a = f.x, bb = f.y, A = f.z;
            const float v00 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, o.x + cb, 0, 0));
            const float v01 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, o.y + cb, 0, 0));
            const float v10 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, o.z + cb, 0, 0));
            const float v11 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, o.w + cb, 0, 0));
            const float wa = 1.f - a, wb = 1.f - bb;
            const float w00 = wa * wb, w01 = a * wb, w10 = wa * bb, w11 = a * bb;
            if (gvalue && live) {
                const float Ag = A * g;
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * w00, gr, o.x + cb, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * w01, gr, o.y + cb, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * w10, gr, o.z + cb, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * w11, gr, o.w + cb, 0, 0);
            }
            const float s = w00 * v00 + w01 * v01 + w10 * v10 + w11 * v11;
            const float dA = lane_sum(g * s, D);
            const float da = lane_sum(g * (wb * (v01 - v00) + bb * (v11 - v10)), D);
            const float db = lane_sum(g * (wa * (v10 - v00) + a * (v11 - v01)), D);
            if (live && c == 0) {
                const int l = i / G.P;
                rec_f[r0 + i] = make_float4(A * da * (float)G.W[l], A * db * (float)G.H[l], A, dA);
            }
        }
    }
    __syncthreads();

    // ---- phase 3: softmax backward, grad_loc and grad_attn
    for (int s = tid; s < nsamp; s += nthr) {
        const int qi = s >> LPlog, i = s & (LP - 1);
        const int q = q0 + qi;
        const bool valid = q < G.q;
        const float4 f = rec_f[s];   // (dL/du, dL/dv, A, dL/dA) for live queries
        float ga = f.w;
        if constexpr (SOFTMAX) {
            const float t = lane_sum(f.z * f.w, LP);
            ga = f.z * (f.w - t);
        }
        if (valid) {
            const long item = ((long)n * G.q + q) * G.m + h;
            if (gloc) *reinterpret_cast<float2*>(gloc + (item * LP + i) * 2) = make_float2(f.x, f.y);
            if (gattn) gattn[item * LP + i] = ga;
        }
    }
}

// Any shape: one lane per (image, query, head), loops over samples and
// channels, global atomics for grad_value.
template <bool SOFTMAX>
__global__ __launch_bounds__(256) void msda_bwd_generic(MsdaGeom G, const float* __restrict__ value,
                                                        const float* __restrict__ loc,
                                                        const float* __restrict__ attn,
                                                        const float* __restrict__ gout, float* __restrict__ gvalue,
                                                        float* __restrict__ gloc, float* __restrict__ gattn)
{
    const long item = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= (long)G.n * G.q * G.m) return;
    const int h = (int)(item % G.m);
    const int n = (int)(item / ((long)G.q * G.m));
    const int LP = G.L * G.P;
    const float* ai = attn + item * LP;
    const float* li = loc + item * LP * 2;
    const float* g = gout + item * G.dh;
    float mx = 0.f, inv = 1.f;
    if (SOFTMAX) {
        mx = ai[0];
        for (int i = 1; i < LP; ++i) mx = fmaxf(mx, ai[i]);
        float s = 0.f;
        for (int i = 0; i < LP; ++i) s += exp_nonpos(ai[i] - mx);
        inv = 1.0f / s;
    }
    const long unit = (long)G.m * G.dh;
    float t = 0.f;   // sum_j A_j dL/dA_j
    for (int pass = 0; pass < (SOFTMAX ? 2 : 1); ++pass) {
        for (int i = 0; i < LP; ++i) {
            const int l = i / G.P;
            const int Hl = G.H[l], Wl = G.W[l];
            const float A = SOFTMAX ? exp_nonpos(ai[i] - mx) * inv : ai[i];
            float dA = 0.f, da = 0.f, db = 0.f;
            const double x = (double)li[2 * i] * Wl - 0.5, y = (double)li[2 * i + 1] * Hl - 0.5;
            if (x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl) {
                const double fx = floor(x), fy = floor(y);
                const float a = (float)(x - fx), b = (float)(y - fy);
                const int x0 = (int)fx, y0 = (int)fy;
                const bool c00 = y0 >= 0 && x0 >= 0, c01 = y0 >= 0 && x0 + 1 < Wl;
                const bool c10 = y0 + 1 < Hl && x0 >= 0, c11 = y0 + 1 < Hl && x0 + 1 < Wl;
                const long base = ((long)n * G.S + G.start[l] + (long)y0 * Wl + x0) * unit + (long)h * G.dh;
                const long rowc = (long)Wl * unit;
                const float wa = 1.f - a, wb = 1.f - b;
                for (int c = 0; c < G.dh; ++c) {
                    const float v00 = c00 ? value[base + c] : 0.f;
                    const float v01 = c01 ? value[base + unit + c] : 0.f;
                    const float v10 = c10 ? value[base + rowc + c] : 0.f;
                    const float v11 = c11 ? value[base + rowc + unit + c] : 0.f;
                    dA += g[c] * (wa * wb * v00 + a * wb * v01 + wa * b * v10 + a * b * v11);
                    da += g[c] * (wb * (v01 - v00) + b * (v11 - v10));
                    db += g[c] * (wa * (v10 - v00) + a * (v11 - v01));
                    if (pass == 0 && gvalue) {
                        const float Ag = A * g[c];
                        if (c00) atomicAdd(gvalue + base + c, Ag * wa * wb);
                        if (c01) atomicAdd(gvalue + base + unit + c, Ag * a * wb);
                        if (c10) atomicAdd(gvalue + base + rowc + c, Ag * wa * b);
                        if (c11) atomicAdd(gvalue + base + rowc + unit + c, Ag * a * b);
                    }
                }
            }
            if (pass == 0) {
                if (gloc) {
                    gloc[(item * LP + i) * 2] = A * da * (float)Wl;
                    gloc[(item * LP + i) * 2 + 1] = A * db * (float)Hl;
                }
                if (SOFTMAX) t += A * dA;
                else if (gattn) gattn[item * LP + i] = dA;
            } else if (gattn) {
                gattn[item * LP + i] = A * (dA - t);
            }
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_f32(float* __restrict__ p, long n)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    if ((uintptr_t)p % 16 == 0) {
        const long n4 = n / 4;
        for (long j = i; j < n4; j += stride) reinterpret_cast<float4*>(p)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (long j = n4 * 4 + i; j < n; j += stride) p[j] = 0.f;
    } else {
        for (long j = i; j < n; j += stride) p[j] = 0.f;
    }
}

}  // namespace

hipError_t launch_msda_backward(const MsdaGeom& G, const float* value, const float* loc, const float* attn,
                                const float* gout, float* gvalue, float* gloc, float* gattn, hipStream_t s)
{
    const long vcount = (long)G.n * G.S * G.m * G.dh;
    if (gvalue) {
        const long blocks = std::min((vcount / 4 + 255) / 256 + 1, 65536L);
        fill_zero_f32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(gvalue, vcount);
    }
    const long items = (long)G.n * G.q * G.m;
    const int LP = G.L * G.P;
    const long value_bytes = vcount * 4;
    const bool aligned = (uintptr_t)loc % 8 == 0 && (!gloc || (uintptr_t)gloc % 8 == 0);
    const bool pow2 = (LP & (LP - 1)) == 0 && LP <= 32 && (G.dh & (G.dh - 1)) == 0 && G.dh <= 64;
    if (aligned && pow2 && value_bytes < (1L << 31) - 64) {
        int LPlog = 0, Dlog = 0;
        while ((1 << LPlog) < LP) ++LPlog;
        while ((1 << Dlog) < G.dh) ++Dlog;
        const int QT = std::min(256 / G.dh, MS_REC_MAX / LP);
        const int tiles = (G.q + QT - 1) / QT;
        const long nwg = (long)G.n * G.m * tiles;
        if (nwg < (1L << 30)) {
            const dim3 grid((unsigned)((nwg + 7) & ~7L)), blk((unsigned)(QT * G.dh));
            if (G.softmax)
                msda_bwd_tile<true><<<grid, blk, 0, s>>>(G, LPlog, Dlog, QT, tiles, (int)nwg, (uint32_t)value_bytes,
                                                         value, loc, attn, gout, gvalue, gloc, gattn);
            else
                msda_bwd_tile<false><<<grid, blk, 0, s>>>(G, LPlog, Dlog, QT, tiles, (int)nwg, (uint32_t)value_bytes,
                                                          value, loc, attn, gout, gvalue, gloc, gattn);
            return hipGetLastError();
        }
    }
    const dim3 grid((unsigned)((items + 255) / 256));
    if (G.softmax)
        msda_bwd_generic<true><<<grid, dim3(256), 0, s>>>(G, value, loc, attn, gout, gvalue, gloc, gattn);
    else
        msda_bwd_generic<false><<<grid, dim3(256), 0, s>>>(G, value, loc, attn, gout, gvalue, gloc, gattn);
    return hipGetLastError();
}

}  // namespace dcn
