// DCN backward kernels for gfx950 (fp32).
//
// The gradients of the forward y_g(p0) = sum_k m_gk x_g(p0 + p_k + dp_gk)
// ("DCNv4: Unbounded Weights", "Why Is Sampling Just 9 Points Still Slow?")
// through the bilinear read, which is differentiable almost everywhere
// ("InternImage: Deformable Convolutions at Scale", Ch.2, "Why bilinear, and
// why it is differentiable").  For tap k with fractions (a, b), corners X_rc
// (row y0+r, column x0+c, zero outside) and output gradient g_c:
//   v_kc          = (1-a)(1-b) X00 + a(1-b) X01 + (1-a) b X10 + a b X11
//   dL/dX_corner += m_k * (corner weight) * g_c          (fp32 atomics)
//   dL/dm_k       = sum_c g_c v_kc
//   dL/ddx_k      = s m_k sum_c g_c [(1-b)(X01-X00) + b(X11-X10)]
//   dL/ddy_k      = s m_k sum_c g_c [(1-a)(X10-X00) + a(X11-X01)]
// and, for DCNv3's softmax ("InternImage...", Ch.3),
//   dL/dz_k = m_k (dL/dm_k - sum_j m_j dL/dm_j).
#include "dcn_device.h"
#include "dcn_bwd_win.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

__global__ __launch_bounds__(256) void fill_zero(float* __restrict__ p, long n)
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

__device__ __forceinline__ float softmax_inputs(const float* mk, int K, float* m, bool softmax)
{
    for (int k = 0; k < K; ++k) m[k] = mk[k];
    if (!softmax) return 0.f;
    float mx = m[0];
    for (int k = 1; k < K; ++k) mx = fmaxf(mx, m[k]);
    float s = 0.f;
    for (int k = 0; k < K; ++k) { m[k] = exp_nonpos(m[k] - mx); s += m[k]; }
    const float inv = 1.0f / s;
    for (int k = 0; k < K; ++k) m[k] *= inv;
    return 0.f;
}

constexpr int KMAX_BWD = 64;   // taps held in registers/scratch per lane

// Sum of v over the P consecutive lanes of an item (P a power of two <= 64).
__device__ __forceinline__ float item_sum(float v, int P)
{
    for (int s = 1; s < P; s <<= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// One lane per (item, CH consecutive channels); P = D / CH lanes per item.
// CH is 4 (16-byte vectors) or 1.
template <int CH, int KH, int KW, bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_bwd_lane(Geom G, const float* __restrict__ x,
                                                    const float* __restrict__ off,
                                                    const float* __restrict__ mask,
                                                    const float* __restrict__ gout, float* __restrict__ gx,
                                                    float* __restrict__ goff, float* __restrict__ gmask)
{
    constexpr int KF = KH * KW;
    const int kh = KH ? KH : G.kh;
    const int K = KF ? KF : G.K;
    const int P = G.d / CH;
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    // Lanes past the end still take part in the shuffles, with no work.
    const bool live = t < (long)G.items * P;
    const int item = live ? (int)(t / P) : 0;
    const int chunk = (int)(t % P);
    const int g = item % G.g;
    const int pix = item / G.g;
    const int wo = pix % G.wo;
    const int nh = pix / G.wo;
    const int ho = nh % G.ho;
    const int n = nh / G.ho;

    float m[KF ? KF : KMAX_BWD];
    softmax_inputs(mask + (long)item * K, K, m, SOFTMAX);
    const float* ob = off + (long)item * K * 2;
    const long img = (long)n * G.h * G.w * G.c + g * G.d + chunk * CH;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;
    const long rowc = (long)G.w * G.c;

    float go[CH];
    if constexpr (CH == 4) {
        load_vec<DT_F32>(gout + (long)item * G.d + chunk * CH, go);
    } else {
        go[0] = gout[(long)item * G.d + chunk];
    }
    if (!live) {
#pragma unroll
        for (int i = 0; i < CH; ++i) go[i] = 0.f;
    }

    float dm[KF ? KF : KMAX_BWD];
    float sdm = 0.f;
#pragma unroll
    for (int kk = 0; kk < K; ++kk) {
        const int kx = kk / kh, ky = kk - kx * kh;
        const float tx = G.scale * ob[2 * kk], ty = G.scale * ob[2 * kk + 1];
        float pm = 0.f, pdx = 0.f, pdy = 0.f;   // this lane's share of the channel sums
        if (live && coord_ok(tx) && coord_ok(ty)) {
            const float fx = floorf(tx), fy = floorf(ty);
            const float a = tx - fx, b = ty - fy;
            const int x0 = bx + kx * G.dw + (int)fx;
            const int y0 = by + ky * G.dh + (int)fy;
            if (x0 >= -1 && x0 < G.w && y0 >= -1 && y0 < G.h) {
                const bool c00 = y0 >= 0 && x0 >= 0, c01 = y0 >= 0 && x0 + 1 < G.w;
                const bool c10 = y0 + 1 < G.h && x0 >= 0, c11 = y0 + 1 < G.h && x0 + 1 < G.w;
                const long base = img + ((long)y0 * G.w + x0) * G.c;
                float X00[CH], X01[CH], X10[CH], X11[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) X00[i] = X01[i] = X10[i] = X11[i] = 0.f;
                if constexpr (CH == 4) {
                    if (c00) load_vec<DT_F32>(x + base, X00);
                    if (c01) load_vec<DT_F32>(x + base + G.c, X01);
                    if (c10) load_vec<DT_F32>(x + base + rowc, X10);
                    if (c11) load_vec<DT_F32>(x + base + rowc + G.c, X11);
                } else {
                    if (c00) X00[0] = x[base];
                    if (c01) X01[0] = x[base + G.c];
                    if (c10) X10[0] = x[base + rowc];
                    if (c11) X11[0] = x[base + rowc + G.c];
                }
                const float wa = 1.f - a, wb = 1.f - b;
                const float w00 = wa * wb, w01 = a * wb, w10 = wa * b, w11 = a * b;
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const float v = w00 * X00[i] + w01 * X01[i] + w10 * X10[i] + w11 * X11[i];
                    pm = fmaf(go[i], v, pm);
                    pdx = fmaf(go[i], wb * (X01[i] - X00[i]) + b * (X11[i] - X10[i]), pdx);
                    pdy = fmaf(go[i], wa * (X10[i] - X00[i]) + a * (X11[i] - X01[i]), pdy);
                }
                if (gx) {
                    const float mk = m[kk];
#pragma unroll
                    for (int i = 0; i < CH; ++i) {
                        const float gi = mk * go[i];
                        if (c00) atomicAdd(gx + base + i, w00 * gi);
                        if (c01) atomicAdd(gx + base + G.c + i, w01 * gi);
                        if (c10) atomicAdd(gx + base + rowc + i, w10 * gi);
                        if (c11) atomicAdd(gx + base + rowc + G.c + i, w11 * gi);
                    }
                }
            }
        }
        const float sm = item_sum(pm, P);
        const float sdx = item_sum(pdx, P);
        const float sdy = item_sum(pdy, P);
        dm[kk] = sm;
        sdm += m[kk] * sm;
        if (live && chunk == 0 && goff) {
            goff[((long)item * K + kk) * 2 + 0] = G.scale * m[kk] * sdx;
            goff[((long)item * K + kk) * 2 + 1] = G.scale * m[kk] * sdy;
        }
    }
    if (live && chunk == 0 && gmask) {
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            gmask[(long)item * K + kk] = SOFTMAX ? m[kk] * (dm[kk] - sdm) : dm[kk];
    }
}

// Any D: one lane per item, channel loop (P = 1, no shuffles).
template <bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_bwd_generic(Geom G, const float* __restrict__ x,
                                                       const float* __restrict__ off,
                                                       const float* __restrict__ mask,
                                                       const float* __restrict__ gout, float* __restrict__ gx,
                                                       float* __restrict__ goff, float* __restrict__ gmask)
{
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= G.items) return;
    const int item = (int)t;
    const int g = item % G.g;
    const int pix = item / G.g;
    const int wo = pix % G.wo;
    const int nh = pix / G.wo;
    const int ho = nh % G.ho;
    const int n = nh / G.ho;
    const int K = G.K;
    float m[KMAX_BWD], dm[KMAX_BWD];
    softmax_inputs(mask + (long)item * K, K, m, SOFTMAX);
    const float* ob = off + (long)item * K * 2;
    const float* go = gout + (long)item * G.d;
    const long img = (long)n * G.h * G.w * G.c + g * G.d;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;
    const long rowc = (long)G.w * G.c;
    float sdm = 0.f;
    for (int kk = 0; kk < K; ++kk) {
        const int kx = kk / G.kh, ky = kk - kx * G.kh;
        const float tx = G.scale * ob[2 * kk], ty = G.scale * ob[2 * kk + 1];
        float sm = 0.f, sdx = 0.f, sdy = 0.f;
        if (coord_ok(tx) && coord_ok(ty)) {
            const float fx = floorf(tx), fy = floorf(ty);
            const float a = tx - fx, b = ty - fy;
            const int x0 = bx + kx * G.dw + (int)fx;
            const int y0 = by + ky * G.dh + (int)fy;
            if (x0 >= -1 && x0 < G.w && y0 >= -1 && y0 < G.h) {
                const bool c00 = y0 >= 0 && x0 >= 0, c01 = y0 >= 0 && x0 + 1 < G.w;
                const bool c10 = y0 + 1 < G.h && x0 >= 0, c11 = y0 + 1 < G.h && x0 + 1 < G.w;
                const long base = img + ((long)y0 * G.w + x0) * G.c;
                const float wa = 1.f - a, wb = 1.f - b;
                const float w00 = wa * wb, w01 = a * wb, w10 = wa * b, w11 = a * b;
                for (int c = 0; c < G.d; ++c) {
                    const float X00 = c00 ? x[base + c] : 0.f;
                    const float X01 = c01 ? x[base + G.c + c] : 0.f;
                    const float X10 = c10 ? x[base + rowc + c] : 0.f;
                    const float X11 = c11 ? x[base + rowc + G.c + c] : 0.f;
                    const float v = w00 * X00 + w01 * X01 + w10 * X10 + w11 * X11;
                    sm = fmaf(go[c], v, sm);
                    sdx = fmaf(go[c], wb * (X01 - X00) + b * (X11 - X10), sdx);
                    sdy = fmaf(go[c], wa * (X10 - X00) + a * (X11 - X01), sdy);
                    if (gx) {
                        const float gi = m[kk] * go[c];
                        if (c00) atomicAdd(gx + base + c, w00 * gi);
                        if (c01) atomicAdd(gx + base + G.c + c, w01 * gi);
                        if (c10) atomicAdd(gx + base + rowc + c, w10 * gi);
                        if (c11) atomicAdd(gx + base + rowc + G.c + c, w11 * gi);
                    }
                }
            }
        }
        dm[kk] = sm;
        sdm += m[kk] * sm;
        if (goff) {
            goff[((long)item * K + kk) * 2 + 0] = G.scale * m[kk] * sdx;
            goff[((long)item * K + kk) * 2 + 1] = G.scale * m[kk] * sdy;
        }
    }
    if (gmask)
        for (int kk = 0; kk < K; ++kk) gmask[(long)item * K + kk] = SOFTMAX ? m[kk] * (dm[kk] - sdm) : dm[kk];
}

// Dispatch.  grad_x is accumulated with fp32 atomics, whose throughput on
// gfx950 scales with the contiguous bytes one instruction adds to (about 21,
// 84 and 330 G adds/s for 4, 16 and 64-byte runs per lane group), so the
// preferred mapping is one lane per channel: the D lanes of an item add to D
// contiguous floats of each corner in one instruction.
template <bool SOFTMAX>
hipError_t launch_typed(const Geom& G, const float* x, const float* off, const float* mask, const float* gout,
                        float* gx, float* goff, float* gmask, hipStream_t s)
{
    const dim3 block(256);
    const bool pow2_1 = G.d <= 64 && (G.d & (G.d - 1)) == 0;
    const bool k_ok = G.K <= KMAX_BWD;
    const long lanes = (long)G.items * G.d;
    if (pow2_1 && G.kh == 3 && G.kw == 3) {
        dcn_bwd_lane<1, 3, 3, SOFTMAX><<<dim3((unsigned)((lanes + 255) / 256)), block, 0, s>>>(
            G, x, off, mask, gout, gx, goff, gmask);
    } else if (pow2_1 && k_ok) {
        dcn_bwd_lane<1, 0, 0, SOFTMAX><<<dim3((unsigned)((lanes + 255) / 256)), block, 0, s>>>(
            G, x, off, mask, gout, gx, goff, gmask);
    } else {
        dcn_bwd_generic<SOFTMAX><<<dim3((unsigned)(((long)G.items + 255) / 256)), block, 0, s>>>(
            G, x, off, mask, gout, gx, goff, gmask);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_backward(const Geom& G, const float* x, const float* off, const float* mask, const float* gout,
                               float* gx, float* goff, float* gmask, hipStream_t s)
{
    if (gx) {
        const long nx = (long)G.n * G.h * G.w * G.c;
        const long blocks = std::min<long>((nx + 255) / 256, 8192);
        fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(gx, nx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // grad_x requested: sum the scatter in LDS (dcn_backward_win.hip)
        // when the window of grad_x rows fits.
        int lds_limit, num_cus;
        device_limits(&lds_limit, &num_cus);
        BwdWinCfg bc;
        if (plan_bwd_win(G, x, gout, lds_limit, num_cus, &bc))
            return launch_dcn_backward_win(G, bc, x, off, mask, gout, gx, goff, gmask, s);
    }
    return G.softmax ? launch_typed<true>(G, x, off, mask, gout, gx, goff, gmask, s)
                     : launch_typed<false>(G, x, off, mask, gout, gx, goff, gmask, s);
}

}  // namespace dcn
