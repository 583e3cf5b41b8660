// DCN backward kernels for gfx950 (f32, f16, bf16 storage; fp32 arithmetic).
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
// grad_x is always summed in fp32: into grad_x itself for f32 storage, else
// into a caller-provided fp32 buffer that is then rounded (to nearest even)
// into the f16/bf16 grad_x.
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

// fp32 sums -> storage type, 8 elements (two 16-byte loads, one 16-byte
// store for f16/bf16) per thread where alignment allows.
template <int DT>
__global__ __launch_bounds__(256) void round_to_storage(const float* __restrict__ src,
                                                        typename Elem<DT>::T* __restrict__ dst, long n)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    const bool vec = (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
    const long n8 = vec ? n / 8 : 0;
    for (long j = i; j < n8; j += stride) {
        float v[8];
        const float4 a = reinterpret_cast<const float4*>(src)[2 * j], b = reinterpret_cast<const float4*>(src)[2 * j + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        store_vec<DT>(dst + 8 * j, v);
    }
    for (long j = n8 * 8 + i; j < n; j += stride) dst[j] = from_f32<DT>(src[j]);
}

template <typename T>
__device__ __forceinline__ float softmax_inputs(const T* mk, int K, float* m, bool softmax)
{
    for (int k = 0; k < K; ++k) m[k] = to_f32(mk[k]);
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

// One lane per (item, channel); P = D lanes per item (a power of two <= 64).
template <int DT, int KH, int KW, bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_bwd_lane(Geom G, const typename Elem<DT>::T* __restrict__ x,
                                                    const typename Elem<DT>::T* __restrict__ off,
                                                    const typename Elem<DT>::T* __restrict__ mask,
                                                    const typename Elem<DT>::T* __restrict__ gout,
                                                    float* __restrict__ gx, typename Elem<DT>::T* __restrict__ goff,
                                                    typename Elem<DT>::T* __restrict__ gmask)
{
    using T = typename Elem<DT>::T;
    constexpr int KF = KH * KW;
    const int kh = KH ? KH : G.kh;
    const int K = KF ? KF : G.K;
    const int P = G.d;
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
    const T* ob = off + (long)item * K * 2;
    const long img = (long)n * G.h * G.w * G.c + g * G.d + chunk;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;
    const long rowc = (long)G.w * G.c;
    const float go = live ? to_f32(gout[(long)item * G.d + chunk]) : 0.f;

    float dm[KF ? KF : KMAX_BWD];
    float sdm = 0.f;
#pragma unroll
    for (int kk = 0; kk < K; ++kk) {
        const int kx = kk / kh, ky = kk - kx * kh;
        const float tx = G.scale * to_f32(ob[2 * kk]), ty = G.scale * to_f32(ob[2 * kk + 1]);
        float pm = 0.f, pdx = 0.f, pdy = 0.f;   // this lane's share of the channel sums
        if (live && coord_ok(tx) && coord_ok(ty)) {
            const float fx = floorf(tx), fy = floorf(ty);
            const float a = tx - fx, b = ty - fy;
            const int x0 = bx + kx * G.dw + (int)fx;
            const int y0 = by + ky * G.dh + (int)fy;
            // px <= -1 or py <= -1 (the edge included), px >= W, py >= H: outside
            if (x0 >= -1 && x0 < G.w && y0 >= -1 && y0 < G.h && !(x0 == -1 && a == 0.f) && !(y0 == -1 && b == 0.f)) {
                const bool c00 = y0 >= 0 && x0 >= 0, c01 = y0 >= 0 && x0 + 1 < G.w;
                const bool c10 = y0 + 1 < G.h && x0 >= 0, c11 = y0 + 1 < G.h && x0 + 1 < G.w;
                const long base = img + ((long)y0 * G.w + x0) * G.c;
                const float X00 = c00 ? to_f32(x[base]) : 0.f;
                const float X01 = c01 ? to_f32(x[base + G.c]) : 0.f;
                const float X10 = c10 ? to_f32(x[base + rowc]) : 0.f;
                const float X11 = c11 ? to_f32(x[base + rowc + G.c]) : 0.f;
                const float wa = 1.f - a, wb = 1.f - b;
                const float w00 = wa * wb, w01 = a * wb, w10 = wa * b, w11 = a * b;
                const float v = w00 * X00 + w01 * X01 + w10 * X10 + w11 * X11;
                pm = go * v;
                pdx = go * (wb * (X01 - X00) + b * (X11 - X10));
                pdy = go * (wa * (X10 - X00) + a * (X11 - X01));
                if (gx) {
                    const float gi = m[kk] * go;
                    if (c00) atomicAdd(gx + base, w00 * gi);
                    if (c01) atomicAdd(gx + base + G.c, w01 * gi);
                    if (c10) atomicAdd(gx + base + rowc, w10 * gi);
                    if (c11) atomicAdd(gx + base + rowc + G.c, w11 * gi);
                }
            }
        }
        const float sm = item_sum(pm, P);
        const float sdx = item_sum(pdx, P);
        const float sdy = item_sum(pdy, P);
        dm[kk] = sm;
        sdm += m[kk] * sm;
        if (live && chunk == 0 && goff) {
            goff[((long)item * K + kk) * 2 + 0] = from_f32<DT>(G.scale * m[kk] * sdx);
            goff[((long)item * K + kk) * 2 + 1] = from_f32<DT>(G.scale * m[kk] * sdy);
        }
    }
    if (live && chunk == 0 && gmask) {
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            gmask[(long)item * K + kk] = from_f32<DT>(SOFTMAX ? m[kk] * (dm[kk] - sdm) : dm[kk]);
    }
}

// Any D: one lane per item, channel loop (P = 1, no shuffles).
template <int DT, bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_bwd_generic(Geom G, const typename Elem<DT>::T* __restrict__ x,
                                                       const typename Elem<DT>::T* __restrict__ off,
                                                       const typename Elem<DT>::T* __restrict__ mask,
                                                       const typename Elem<DT>::T* __restrict__ gout,
                                                       float* __restrict__ gx, typename Elem<DT>::T* __restrict__ goff,
                                                       typename Elem<DT>::T* __restrict__ gmask)
{
    using T = typename Elem<DT>::T;
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
    const T* ob = off + (long)item * K * 2;
    const T* go = gout + (long)item * G.d;
    const long img = (long)n * G.h * G.w * G.c + g * G.d;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;
    const long rowc = (long)G.w * G.c;
    float sdm = 0.f;
    for (int kk = 0; kk < K; ++kk) {
        const int kx = kk / G.kh, ky = kk - kx * G.kh;
        const float tx = G.scale * to_f32(ob[2 * kk]), ty = G.scale * to_f32(ob[2 * kk + 1]);
        float sm = 0.f, sdx = 0.f, sdy = 0.f;
        if (coord_ok(tx) && coord_ok(ty)) {
            const float fx = floorf(tx), fy = floorf(ty);
            const float a = tx - fx, b = ty - fy;
            const int x0 = bx + kx * G.dw + (int)fx;
            const int y0 = by + ky * G.dh + (int)fy;
            // px <= -1 or py <= -1 (the edge included), px >= W, py >= H: outside
            if (x0 >= -1 && x0 < G.w && y0 >= -1 && y0 < G.h && !(x0 == -1 && a == 0.f) && !(y0 == -1 && b == 0.f)) {
                const bool c00 = y0 >= 0 && x0 >= 0, c01 = y0 >= 0 && x0 + 1 < G.w;
                const bool c10 = y0 + 1 < G.h && x0 >= 0, c11 = y0 + 1 < G.h && x0 + 1 < G.w;
                const long base = img + ((long)y0 * G.w + x0) * G.c;
                const float wa = 1.f - a, wb = 1.f - b;
                const float w00 = wa * wb, w01 = a * wb, w10 = wa * b, w11 = a * b;
                for (int c = 0; c < G.d; ++c) {
                    const float X00 = c00 ? to_f32(x[base + c]) : 0.f;
                    const float X01 = c01 ? to_f32(x[base + G.c + c]) : 0.f;
                    const float X10 = c10 ? to_f32(x[base + rowc + c]) : 0.f;
                    const float X11 = c11 ? to_f32(x[base + rowc + G.c + c]) : 0.f;
                    const float gc = to_f32(go[c]);
                    const float v = w00 * X00 + w01 * X01 + w10 * X10 + w11 * X11;
                    sm = fmaf(gc, v, sm);
                    sdx = fmaf(gc, wb * (X01 - X00) + b * (X11 - X10), sdx);
                    sdy = fmaf(gc, wa * (X10 - X00) + a * (X11 - X01), sdy);
                    if (gx) {
                        const float gi = m[kk] * gc;
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
            goff[((long)item * K + kk) * 2 + 0] = from_f32<DT>(G.scale * m[kk] * sdx);
            goff[((long)item * K + kk) * 2 + 1] = from_f32<DT>(G.scale * m[kk] * sdy);
        }
    }
    if (gmask)
        for (int kk = 0; kk < K; ++kk)
            gmask[(long)item * K + kk] = from_f32<DT>(SOFTMAX ? m[kk] * (dm[kk] - sdm) : dm[kk]);
}

// Dispatch of the fallbacks.  grad_x is accumulated with fp32 atomics,
// whose throughput on gfx950 scales with the contiguous bytes one
// instruction adds to (about 21, 84 and 330 G adds/s for 4, 16 and 64-byte
// runs per lane group), so the preferred mapping is one lane per channel:
// the D lanes of an item add to D contiguous floats of each corner in one
// instruction.
template <int DT, bool SOFTMAX>
hipError_t launch_typed(const Geom& G, const void* x, const void* off, const void* mask, const void* gout,
                        float* gx, void* goff, void* gmask, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const dim3 block(256);
    const bool pow2_1 = G.d <= 64 && (G.d & (G.d - 1)) == 0;
    const bool k_ok = G.K <= KMAX_BWD;
    const long lanes = (long)G.items * G.d;
    const T *xt = (const T*)x, *ot = (const T*)off, *mt = (const T*)mask, *gt = (const T*)gout;
    if (pow2_1 && G.kh == 3 && G.kw == 3) {
        dcn_bwd_lane<DT, 3, 3, SOFTMAX><<<dim3((unsigned)((lanes + 255) / 256)), block, 0, s>>>(
            G, xt, ot, mt, gt, gx, (T*)goff, (T*)gmask);
    } else if (pow2_1 && k_ok) {
        dcn_bwd_lane<DT, 0, 0, SOFTMAX><<<dim3((unsigned)((lanes + 255) / 256)), block, 0, s>>>(
            G, xt, ot, mt, gt, gx, (T*)goff, (T*)gmask);
    } else {
        dcn_bwd_generic<DT, SOFTMAX><<<dim3((unsigned)(((long)G.items + 255) / 256)), block, 0, s>>>(
            G, xt, ot, mt, gt, gx, (T*)goff, (T*)gmask);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dtype(const Geom& G, const void* x, const void* off, const void* mask, const void* gout,
                        void* gx, void* goff, void* gmask, float* ws, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    // Where grad_x is summed: grad_x itself for f32, else the fp32 buffer.
    float* sum = DT == DT_F32 ? (float*)gx : (gx ? ws : nullptr);
    const long nx = (long)G.n * G.h * G.w * G.c;
    hipError_t e = hipSuccess;
    if (sum) {
        const long blocks = std::min<long>((nx + 255) / 256, 8192);
        fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(sum, nx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // With grad_x requested, sum the scatter in LDS (dcn_backward_win.hip)
    // when the window of grad_x rows fits.
    int lds_limit, num_cus;
    device_limits(&lds_limit, &num_cus);
    BwdWinCfg bc;
    if (sum && plan_bwd_win(G, DT, x, gout, lds_limit, num_cus, &bc))
        e = launch_dcn_backward_win(G, bc, DT, x, off, mask, gout, sum, goff, gmask, s);
    else
        e = G.softmax ? launch_typed<DT, true>(G, x, off, mask, gout, sum, goff, gmask, s)
                      : launch_typed<DT, false>(G, x, off, mask, gout, sum, goff, gmask, s);
    if (e != hipSuccess) return e;
    if constexpr (DT != DT_F32) {
        if (sum) {
            const long blocks = std::min<long>((nx / 8 + 255) / 256 + 1, 8192);
            round_to_storage<DT><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(sum, (T*)gx, nx);
            e = hipGetLastError();
        }
    }
    return e;
}

}  // namespace

hipError_t launch_dcn_backward(const Geom& G, int dtype, const void* x, const void* off, const void* mask,
                               const void* gout, void* gx, void* goff, void* gmask, float* ws, hipStream_t s)
{
    switch (dtype) {
        case DT_F32: return launch_dtype<DT_F32>(G, x, off, mask, gout, gx, goff, gmask, ws, s);
        case DT_F16: return launch_dtype<DT_F16>(G, x, off, mask, gout, gx, goff, gmask, ws, s);
        case DT_BF16: return launch_dtype<DT_BF16>(G, x, off, mask, gout, gx, goff, gmask, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
