// DCN forward kernels for gfx950.
//
// The operator ("DCNv4: Unbounded Weights", "Why Is Sampling Just 9 Points
// Still Slow?"): for output pixel p0 and channel group g,
//     y_g(p0) = sum_k m_gk * x_g(p0 + p_k + dp_gk)
// where x_g(p) is the bilinear read of the group's D channels at the
// fractional point p, zero outside the map ("InternImage: Deformable
// Convolutions at Scale", Ch.2), and m_gk is softmax-normalised over the K
// taps for DCNv3 (same page, Ch.3) or used as given for DCNv4 ("DCNv4:
// Unbounded Weights", "1. Remove Softmax").
//
// Work item = one (output pixel, group).  The per-tap geometry (floor,
// fraction, four corner weights premultiplied by m, validity) is computed
// once per item and tap and reused for every channel the lane holds; corner
// reads are 16-byte vector loads along the NHWC channel axis; accumulation is
// fp32; there are no atomics (each output element has exactly one writer).
#include "dcn_device.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

// Modulation of the K taps of one item: softmax over K (max subtracted) or
// the values as given.  KF > 0 keeps them in registers.
template <int DT, int KF, bool SOFTMAX>
struct Modulation {
    using T = typename Elem<DT>::T;
    float m[KF];
    __device__ __forceinline__ void init(const T* mk, int /*K*/)
    {
#pragma unroll
        for (int k = 0; k < KF; ++k) m[k] = to_f32(mk[k]);
        if constexpr (SOFTMAX) {
            float mx = m[0];
#pragma unroll
            for (int k = 1; k < KF; ++k) mx = fmaxf(mx, m[k]);
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < KF; ++k) { m[k] = exp_nonpos(m[k] - mx); s += m[k]; }
            float inv = 1.0f / s;
#pragma unroll
            for (int k = 0; k < KF; ++k) m[k] *= inv;
        }
    }
    __device__ __forceinline__ float operator()(int k) const { return m[k]; }
};

template <int DT, bool SOFTMAX>
struct Modulation<DT, 0, SOFTMAX> {
    using T = typename Elem<DT>::T;
    const T* mk;
    float mx, inv;
    __device__ __forceinline__ void init(const T* p, int K)
    {
        mk = p;
        if constexpr (SOFTMAX) {
            mx = to_f32(p[0]);
            for (int k = 1; k < K; ++k) mx = fmaxf(mx, to_f32(p[k]));
            float s = 0.f;
            for (int k = 0; k < K; ++k) s += exp_nonpos(to_f32(p[k]) - mx);
            inv = 1.0f / s;
        }
    }
    __device__ __forceinline__ float operator()(int k) const
    {
        if constexpr (SOFTMAX) return exp_nonpos(to_f32(mk[k]) - mx) * inv;
        return to_f32(mk[k]);
    }
};

// Geometry of one tap: corner weights already multiplied by the modulation,
// zero for a corner outside the map (`in` bit q set for a corner inside);
// `base` points at the top-left corner.
struct Tap {
    float w00, w01, w10, w11;
    long base;       // element index of corner (y0, x0), channel 0 of the image
    bool any;
    unsigned in;     // bit q: corner q (00, 01, 10, 11) lies inside the map
};

__device__ __forceinline__ Tap tap_geometry(const Geom& G, int bx, int by, int kx, int ky, float dx, float dy,
                                            float m)
{
    Tap t;
    t.any = false;
    const float tx = G.scale * dx, ty = G.scale * dy;
    if (!(coord_ok(tx) && coord_ok(ty))) return t;
    const float fx = floorf(tx), fy = floorf(ty);
    const float a = tx - fx, b = ty - fy;
    const int x0 = bx + kx * G.dw + (int)fx;
    const int y0 = by + ky * G.dh + (int)fy;
    if (x0 < -1 || x0 >= G.w || y0 < -1 || y0 >= G.h) return t;
    const bool cx0 = x0 >= 0, cx1 = x0 + 1 < G.w, cy0 = y0 >= 0, cy1 = y0 + 1 < G.h;
    const float ma = m * (1.f - a), mb = m * a;
    t.w00 = (cy0 && cx0) ? ma * (1.f - b) : 0.f;
    t.w01 = (cy0 && cx1) ? mb * (1.f - b) : 0.f;
    t.w10 = (cy1 && cx0) ? ma * b : 0.f;
    t.w11 = (cy1 && cx1) ? mb * b : 0.f;
    t.base = ((long)y0 * G.w + x0) * G.c;
    t.any = true;
    t.in = (cy0 && cx0 ? 1u : 0u) | (cy0 && cx1 ? 2u : 0u) | (cy1 && cx0 ? 4u : 0u) | (cy1 && cx1 ? 8u : 0u);
    return t;
}

// Byte offsets of the four corners of one tap inside the x buffer, and their
// weights premultiplied by the modulation.  A corner outside the map gets an
// offset past the end of the buffer, which the buffer load returns as zero:
// that is the zero padding, with no branch and no clamped address.
struct TapV {
    float w00, w01, w10, w11;
    uint32_t o00, o01, o10, o11;
};

constexpr uint32_t OOB = 0x80000000u;   // beyond any x accepted on this path (< 2^31 bytes)

__device__ __forceinline__ TapV tap_vec(const Geom& G, int bx, int by, int kx, int ky, float dx, float dy, float m,
                                        uint32_t lane_base, uint32_t pix_bytes, uint32_t row_bytes)
{
    // Clamp keeps floor/int conversion defined; NaN becomes -2^24 (fmaxf picks
    // the number), far outside any map.
    const float lim = 16777216.0f;
    const float tx = fminf(fmaxf(G.scale * dx, -lim), lim);
    const float ty = fminf(fmaxf(G.scale * dy, -lim), lim);
    const float fx = floorf(tx), fy = floorf(ty);
    const float a = tx - fx, b = ty - fy;
    const int x0 = bx + kx * G.dw + (int)fx;
    const int y0 = by + ky * G.dh + (int)fy;
    const bool cx0 = (unsigned)x0 < (unsigned)G.w, cx1 = (unsigned)(x0 + 1) < (unsigned)G.w;
    const bool cy0 = (unsigned)y0 < (unsigned)G.h, cy1 = (unsigned)(y0 + 1) < (unsigned)G.h;
    const uint32_t base = lane_base + ((uint32_t)y0 * (uint32_t)G.w + (uint32_t)x0) * pix_bytes;
    TapV t;
    const float ma = m * (1.f - a), mb = m * a;
    t.w00 = ma * (1.f - b);
    t.w01 = mb * (1.f - b);
    t.w10 = ma * b;
    t.w11 = mb * b;
    t.o00 = (cy0 && cx0) ? base : OOB;
    t.o01 = (cy0 && cx1) ? base + pix_bytes : OOB;
    t.o10 = (cy1 && cx0) ? base + row_bytes : OOB;
    t.o11 = (cy1 && cx1) ? base + row_bytes + pix_bytes : OOB;
    return t;
}

template <int DT>
__device__ __forceinline__ void fma_corner(float* acc, float w, u32x4 r)
{
    constexpr int V = Vec<DT>::N;
    float v[V];
    if constexpr (DT == DT_F32) {
        v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
    } else {
        const uint32_t q[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DT_F16) {
                v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i] & 0xffffu));
                v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i] >> 16));
            } else {
                v[2 * i] = __uint_as_float(q[i] << 16);
                v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(w, v[i], acc[i]);
}

// One lane per (item, 16-byte channel vector); P = D / V lanes per item.
// x is read through a buffer resource covering the whole tensor (< 2^31 bytes).
template <int DT, int KH, int KW, bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_fwd_vec(Geom G, const typename Elem<DT>::T* __restrict__ x,
                                                   const typename Elem<DT>::T* __restrict__ off,
                                                   const typename Elem<DT>::T* __restrict__ mask,
                                                   typename Elem<DT>::T* __restrict__ out, uint32_t x_bytes)
{
    using T = typename Elem<DT>::T;
    constexpr int V = Vec<DT>::N;
    constexpr int KF = KH * KW;
    const int kh = KH ? KH : G.kh;
    const int K = KF ? KF : G.K;
    const int P = G.d / V;
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int item = (int)(t / P);
    if (item >= G.items) return;
    const int chunk = (int)(t - (long)item * P);
    const int g = item % G.g;
    const int pix = item / G.g;
    const int wo = pix % G.wo;
    const int nh = pix / G.wo;
    const int ho = nh % G.ho;
    const int n = nh / G.ho;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, 0x00020000);
    Modulation<DT, KF, SOFTMAX> mod;
    mod.init(mask + (long)item * K, K);
    const T* ob = off + (long)item * K * 2;
    const uint32_t es = sizeof(T);
    const uint32_t lane_base = ((uint32_t)n * G.h * G.w * G.c + g * G.d + chunk * V) * es;
    const uint32_t pix_bytes = (uint32_t)G.c * es, row_bytes = (uint32_t)G.w * G.c * es;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

#pragma unroll
    for (int kk = 0; kk < K; ++kk) {
        const int kx = kk / kh, ky = kk - kx * kh;
        const TapV tp = tap_vec(G, bx, by, kx, ky, to_f32(ob[2 * kk]), to_f32(ob[2 * kk + 1]), mod(kk), lane_base,
                                pix_bytes, row_bytes);
        const u32x4 r00 = __builtin_amdgcn_raw_buffer_load_b128(xr, tp.o00, 0, 0);
        const u32x4 r01 = __builtin_amdgcn_raw_buffer_load_b128(xr, tp.o01, 0, 0);
        const u32x4 r10 = __builtin_amdgcn_raw_buffer_load_b128(xr, tp.o10, 0, 0);
        const u32x4 r11 = __builtin_amdgcn_raw_buffer_load_b128(xr, tp.o11, 0, 0);
        fma_corner<DT>(acc, tp.w00, r00);
        fma_corner<DT>(acc, tp.w01, r01);
        fma_corner<DT>(acc, tp.w10, r10);
        fma_corner<DT>(acc, tp.w11, r11);
    }
    store_vec<DT>(out + (long)item * G.d + chunk * V, acc);
}

// Any D and element alignment: one lane per item, scalar channel loop.
template <int DT, bool SOFTMAX>
__global__ __launch_bounds__(256) void dcn_fwd_generic(Geom G, const typename Elem<DT>::T* __restrict__ x,
                                                       const typename Elem<DT>::T* __restrict__ off,
                                                       const typename Elem<DT>::T* __restrict__ mask,
                                                       typename Elem<DT>::T* __restrict__ out)
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
    Modulation<DT, 0, SOFTMAX> mod;
    mod.init(mask + (long)item * K, K);
    const T* ob = off + (long)item * K * 2;
    const T* xb = x + (long)n * G.h * G.w * G.c + g * G.d;
    T* ob_out = out + (long)item * G.d;
    const int bx = wo * G.sw - G.pw, by = ho * G.sh - G.ph;
    const long rowc = (long)G.w * G.c;
    for (int c0 = 0; c0 < G.d; c0 += 8) {
        const int nc = min(8, G.d - c0);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            const int kx = kk / G.kh, ky = kk - kx * G.kh;
            const Tap tp = tap_geometry(G, bx, by, kx, ky, to_f32(ob[2 * kk]), to_f32(ob[2 * kk + 1]), mod(kk));
            if (!tp.any) continue;
            const T* r = xb + tp.base + c0;
            const float w[4] = {tp.w00, tp.w01, tp.w10, tp.w11};
            const long o[4] = {0, G.c, rowc, rowc + G.c};
            for (int q = 0; q < 4; ++q) {
                // a corner outside the map is skipped; one inside is summed
                // even at weight zero (0 * non-finite x is NaN, as in the sum's definition)
                if (!(tp.in >> q & 1u)) continue;
                for (int i = 0; i < nc; ++i) acc[i] = fmaf(w[q], to_f32(r[o[q] + i]), acc[i]);
            }
        }
        for (int i = 0; i < nc; ++i) {
            ob_out[c0 + i] = from_f32<DT>(acc[i]);
            count_writes(ob_out + c0 + i, 1);
        }
    }
}

template <int DT, bool SOFTMAX>
hipError_t launch_typed(const Geom& G, const void* x, const void* off, const void* mask, void* out, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    constexpr int V = Vec<DT>::N;
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)out % 16 == 0);
    const int P = G.d / V;
    const long x_bytes = (long)G.n * G.h * G.w * G.c * (long)sizeof(T);
    if (aligned && G.d % V == 0 && x_bytes < (long)OOB) {
        const long lanes = (long)G.items * P;
        const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
        if (G.kh == 3 && G.kw == 3)
            dcn_fwd_vec<DT, 3, 3, SOFTMAX><<<grid, block, 0, s>>>(G, (const T*)x, (const T*)off, (const T*)mask,
                                                                   (T*)out, (uint32_t)x_bytes);
        else
            dcn_fwd_vec<DT, 0, 0, SOFTMAX><<<grid, block, 0, s>>>(G, (const T*)x, (const T*)off, (const T*)mask,
                                                                   (T*)out, (uint32_t)x_bytes);
    } else {
        const dim3 grid((unsigned)(((long)G.items + 255) / 256)), block(256);
        dcn_fwd_generic<DT, SOFTMAX><<<grid, block, 0, s>>>(G, (const T*)x, (const T*)off, (const T*)mask, (T*)out);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_forward(const Geom& G, int dtype, const void* x, const void* off, const void* mask, void* out,
                              hipStream_t s)
{
    int lds_limit, num_cus;
    device_limits(&lds_limit, &num_cus);
    // The LDS sliding-window kernel where it applies, else the direct gathers.
    RingCfg rr;
    Geom gk;
    if (plan_ring(G, dtype, x, off, mask, out, lds_limit, num_cus, &rr, &gk))
        return launch_dcn_forward_ring(gk, rr, dtype, x, off, mask, out, s);
    switch (dtype * 2 + (G.softmax ? 1 : 0)) {
        case DT_F32 * 2 + 0: return launch_typed<DT_F32, false>(G, x, off, mask, out, s);
        case DT_F32 * 2 + 1: return launch_typed<DT_F32, true>(G, x, off, mask, out, s);
        case DT_F16 * 2 + 0: return launch_typed<DT_F16, false>(G, x, off, mask, out, s);
        case DT_F16 * 2 + 1: return launch_typed<DT_F16, true>(G, x, off, mask, out, s);
        case DT_BF16 * 2 + 0: return launch_typed<DT_BF16, false>(G, x, off, mask, out, s);
        case DT_BF16 * 2 + 1: return launch_typed<DT_BF16, true>(G, x, off, mask, out, s);
    }
    return hipErrorInvalidValue;
}

#ifdef DCN_COUNT_WRITES
DCN_WRITE_COUNT_SETTER(fwd_count_writes)
#endif

}  // namespace dcn
