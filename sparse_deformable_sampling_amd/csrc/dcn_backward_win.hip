// DCN backward with grad_x accumulated on chip, for gfx950 (f32, f16, bf16
// storage; fp32 arithmetic, and grad_x summed in fp32).
//
// The gradients are those of dcn_backward.hip (the derivative of y_g(p0) =
// sum_k m_gk x_g(p0 + p_k + dp_gk), "DCNv4: Unbounded Weights", "Why Is
// Sampling Just 9 Points Still Slow?", through the bilinear read of
// "InternImage: Deformable Convolutions at Scale", Ch.2).  What differs is
// how the scatter into grad_x is summed.
//
// fp32 atomics into global memory are served at about 21 G requests of up to
// 64 bytes per second on this chip, so scattering 36 corner contributions per
// (pixel, group, channel) straight to grad_x is bound by them.  LDS integer
// atomics run about twenty times faster (ds_add_u64 ~7 lanes/clk/CU), LDS
// float atomics do not (ds_add_f32 ~0.3 lanes/clk/CU).  So each workgroup
// owns one image, one channel group and a chunk of output rows, walks down
// the chunk a few rows per step, and keeps a window of grad_x rows of its
// group in LDS as 64-bit fixed-point sums:
//  - a contribution v to a cell whose row is in the window is added as
//    round(v * 2^e), sign-extended to 64 bits, with ds_add_u64; its row leaves the window once no
//    later output row of the chunk can reach it through LDS, and is then
//    converted back to fp32 and added to grad_x with one fp32 atomic per
//    element (neighbouring chunks share halo rows);
//  - a contribution to a row outside the window (an offset beyond the halo)
//    goes to grad_x with an fp32 atomic directly.
// The scale 2^e is chosen per workgroup from the item bounds
// b = max_k |m_k| * max_c |g_c|, which no single contribution m_k w g_c
// (w <= 1) of that item can exceed.  A pre-scan counts the workgroup's items
// per binary exponent of b (one item in eight, spread over the chunk: the
// bound only sets the resolution, since any tap above B is routed to the
// atomics) and takes for B = 2^E the smaller of the least
// power of two that bounds all but about one item in a thousand and 64 times
// the median item's bound (the margin keeps items of ordinary spread under
// B, the median keeps outliers from setting it): e makes B * 2^e = 2^30,
// so one contribution below B is one 32-bit integer (a single conversion),
// resolving 2^-30 of B, and a cell's 64-bit sum of fewer than 2^32 of them
// cannot overflow.  A lane whose tap could reach B (|m_k| times the largest
// |g_c| of its channels) sends that tap's contributions to grad_x with fp32
// atomics instead, so a few large modulations (DCNv4's are unbounded) do not
// coarsen the rest of the workgroup's sums.  A tap whose |m_k| or any of the
// lane's |g_c| is not finite fails that test too (its bound is NaN or Inf),
// so non-finite values reach grad_x through fp32 atomics as they would
// through any sum; non-finite values in the sampled items, or a B outside
// [2^-59, 2^60], turn the fixed-point path off for the whole workgroup.
// Integer sums do not depend on the order of the additions.
// With f16/bf16 storage the inputs are widened to fp32 as they are read,
// grad_offset and grad_mask are rounded once (to nearest even) as they are
// stored, and grad_x is summed into an fp32 buffer that the caller converts.
#include <algorithm>

#include "dcn_device.h"
#include "dcn_bwd_win.h"

namespace dcn {

namespace {

constexpr uint32_t OOB = 0x80000000u;
constexpr int KMAX_WIN = 64;

// Sum of v over aligned groups of `width` lanes (a power of two).  Partners
// 1 and 2 apart are read with DPP quad permutations, which stay in the VALU;
// __shfl_xor would go through the LDS crossbar (ds_bpermute) and wait behind
// the wave's queued LDS atomics on every tap.
__device__ __forceinline__ float lane_sum(float v, int width)
{
    if (width > 1) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    if (width > 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    for (int o = 4; o < width; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Fixed-point image of t (|t| < 2^30): t rounded to a nearest integer (ties
// up; within one unit where t + 1/2 is not exact), as a two's-complement
// 64-bit integer.  One conversion instruction, floor(t + 1/2) to int32, where
// rounding and converting separately take two; the compiler does not form it
// from C, hence the one-instruction VALU asm (no memory access).
__device__ __forceinline__ unsigned long long to_fixed(float t)
{
    int r;
    asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(t));
    return (unsigned long long)(long long)r;
}

// RW consecutive dwords at p (RW a multiple of 4, or 2; p 16- or 8-byte aligned).
template <int RW, typename T>
__device__ __forceinline__ void load_words(const T* p, uint32_t* w)
{
    if constexpr (RW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < RW / 4; ++i) {
            const u32x4 r = reinterpret_cast<const u32x4*>(p)[i];
            w[4 * i] = r.x; w[4 * i + 1] = r.y; w[4 * i + 2] = r.z; w[4 * i + 3] = r.w;
        }
    } else {
        static_assert(RW == 2, "8 or a multiple of 16 bytes");
        const uint2 r = *reinterpret_cast<const uint2*>(p);
        w[0] = r.x; w[1] = r.y;
    }
}

// The RW dwords holding a lane's CPL channels of one corner, widened to fp32.
template <int DT, int CPL>
__device__ __forceinline__ void widen(const uint32_t* w, float* v)
{
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        if constexpr (DT == DT_F32) v[j] = __uint_as_float(w[j]);
        else if constexpr (DT == DT_F16)
            v[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? w[j >> 1] >> 16 : w[j >> 1] & 0xffffu));
        else v[j] = __uint_as_float((j & 1) ? w[j >> 1] & 0xffff0000u : w[j >> 1] << 16);
    }
}

// Sum over a lane's CPL channels of g_c * X_c, with X_c one corner's channels
// as loaded (RW dwords of the storage type) and g_c grad_out: in fp32 as
// widened floats (gf), and for f16/bf16 straight from the packed pairs (gp)
// with the two-product dot instructions, whose products are exact in fp32 and
// which sum in fp32.
template <int DT, int CPL>
__device__ __forceinline__ float corner_dot(const uint32_t* w, const float* gf, const uint32_t* gp)
{
    constexpr int RW = CPL * (int)sizeof(typename Elem<DT>::T) / 4;
    float s = 0.f;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) s = fmaf(gf[j], __uint_as_float(w[j]), s);
    } else if constexpr (DT == DT_F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < RW; ++i)
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w[i]), __builtin_bit_cast(h2, gp[i]), s, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < RW; ++i)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w[i]), __builtin_bit_cast(b2, gp[i]), s, false);
    }
    return s;
}

// Buffer loads of RW dwords at byte offset o (an offset past the buffer reads zero).
template <int RW>
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rs, uint32_t o, uint32_t* w)
{
    if constexpr (RW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < RW / 4; ++i) {
            const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 16u * i, 0, 0);
            w[4 * i] = r.x; w[4 * i + 1] = r.y; w[4 * i + 2] = r.z; w[4 * i + 3] = r.w;
        }
    } else {
        static_assert(RW == 2, "8 or a multiple of 16 bytes");
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 r = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
        w[0] = r.x; w[1] = r.y;
    }
}

// DT = storage type of x, offset, mask, grad_out, grad_offset and grad_mask
// (grad_x is fp32).  NV: a lane holds 4 NV channels; a (pixel, group) item
// has D / (4 NV) lanes.
template <int DT, int KH, int KW, bool SOFTMAX, int NV>
__global__ __launch_bounds__(512) void dcn_bwd_win(Geom G, BwdWinCfg bc, const typename Elem<DT>::T* __restrict__ x,
                                                   const typename Elem<DT>::T* __restrict__ off,
                                                   const typename Elem<DT>::T* __restrict__ mask,
                                                   const typename Elem<DT>::T* __restrict__ gout,
                                                   float* __restrict__ gx, typename Elem<DT>::T* __restrict__ goff,
                                                   typename Elem<DT>::T* __restrict__ gmask)
{
    using T = typename Elem<DT>::T;
    constexpr int ES = (int)sizeof(T);
    constexpr int KF = KH * KW;
    extern __shared__ unsigned long long acc[];   // [aw][w][d] fixed-point sums
    __shared__ int red_bad[16];
    __shared__ int hist[128];                     // items per binary exponent of their bound, + 63
    __shared__ int E_s;
    const int K = KF ? KF : G.K;
    const int kh = KH ? KH : G.kh;
    const int tid = threadIdx.x, nthr = blockDim.x;
    int L = blockIdx.x;
    if (bc.nwg % 8 == 0) L = (blockIdx.x % 8) * (bc.nwg / 8) + blockIdx.x / 8;   // neighbours share an XCD
    const int chunk = L % bc.chunks;
    const int ng = L / bc.chunks;
    const int g = ng % G.g, n = ng / G.g;
    const int r_begin = chunk * bc.chunk_rows;
    const int r_end = min(G.ho, r_begin + bc.chunk_rows);
    if (r_begin >= r_end) return;
    const int D = G.d, C = G.c, W = G.w, H = G.h;
    constexpr int CPL = 4 * NV;                      // channels per lane
    constexpr int RW = CPL * ES / 4;                 // dwords of a lane's channels of one corner
    const int d_log = bc.lq_log + 2 + (NV == 2);     // D = CPL * lanes per item, a power of two
    // A window row holds W pixels of D sums at a stride of D + 1 words: the
    // odd stride spreads a wave's atomics over the LDS banks (with a
    // power-of-two stride all of them would fall on a few).
    const int pstr = D + 1;
    const int rowe = W * pstr;                       // 8-byte words of one window row
    const int wlo0 = r_begin * G.sh - G.ph - bc.hy - 1;
    const int lq = 1 << bc.lq_log;
    const int li = tid >> bc.lq_log, c4 = tid & (lq - 1);

    // ---- the bound B of this workgroup, and whether every input is finite
    for (int i = tid; i < 128; i += nthr) hist[i] = 0;
    __syncthreads();
    int bad = 0;
    // Same lane layout as the main pass: lane (item, chunk) reads its CPL
    // channels of grad_out with 16-byte loads and every lq-th logit.
    const int nitems = (r_end - r_begin) * G.wo;
    constexpr int SAMPLE = 8;         // one item in SAMPLE
    for (int it0 = 0; it0 * SAMPLE < nitems; it0 += bc.ip) {
        const int it = (it0 + li) * SAMPLE;
        if (it >= nitems) continue;   // whole items only: the reductions below stay within one item
        const long pix = ((long)n * G.ho + r_begin + it / G.wo) * G.wo + it % G.wo;
        const long item = pix * G.g + g;
        float ms = 0.f;
        for (int k = c4; k < K; k += lq) {
            const float v = to_f32(mask[item * K + k]);
            ms = fmaxf(ms, fabsf(v));
            bad |= !(fabsf(v) <= 3.0e38f);
        }
        float gm = 0.f;
        {
            float a[CPL];
            uint32_t w[RW];
            load_words<RW>(gout + pix * C + (long)g * D + CPL * c4, w);
            widen<DT, CPL>(w, a);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                gm = fmaxf(gm, fabsf(a[j]));
                bad |= !(fabsf(a[j]) <= 3.0e38f);
            }
        }
        for (int o = 1; o < lq; o <<= 1) {
            ms = fmaxf(ms, __shfl_xor(ms, o, 64));
            gm = fmaxf(gm, __shfl_xor(gm, o, 64));
        }
        if (SOFTMAX) ms = 1.f;
        if (c4 == 0) {
            int ex = 0;
            (void)frexpf(ms * gm, &ex);      // b < 2^ex (ex = 0 for b = 0)
            atomicAdd(&hist[min(max(ex + 63, 0), 127)], 1);
        }
    }
    for (int o = 1; o < 64; o <<= 1) bad |= __shfl_xor(bad, o, 64);
    if ((tid & 63) == 0) red_bad[tid >> 6] = bad;
    __syncthreads();
    bad = 0;
    for (int w = 0; w < (nthr + 63) / 64; ++w) bad |= red_bad[w];
    // B = 2^E, from the histogram by one wave (lane i holds bins 2i, 2i+1;
    // cum(b) = items in bins <= b, non-decreasing in b):
    //   top: the least bin b with at most `allow` items above it;
    //   med: the least bin b with cum(b) >= half of the items.
    if (tid < 64) {
        const int h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
        int incl = h0 + h1;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (tid >= o) incl += t;
        }
        const int total = __shfl(incl, 63, 64);
        const int cum0 = incl - h1, cum1 = incl;   // cum(2i), cum(2i+1)
        const int allow = total >> 10, half = (total + 1) / 2;
        // bin 127 satisfies both tests, so every ballot below has a set bit
        const unsigned long long t0 = __ballot(total - cum0 <= allow), t1 = __ballot(total - cum1 <= allow);
        const unsigned long long q0 = __ballot(cum0 >= half), q1 = __ballot(cum1 >= half);
        auto least = [](unsigned long long even, unsigned long long odd) {
            const int be = even ? 2 * __builtin_ctzll(even) : 128, bo = odd ? 2 * __builtin_ctzll(odd) + 1 : 128;
            return min(be, bo);
        };
        if (tid == 0) E_s = min(least(t0, t1), least(q0, q1) + 6) - 63;
    }
    for (int i = tid; i < bc.aw * rowe; i += nthr) acc[i] = 0ull;
    __syncthreads();
    const int E = E_s;
    const bool fixed = !bad && E >= -59 && E <= 60;
    const float Bf = ldexpf(1.f, E);        // a tap of a lane reaching this takes the atomics
    const int e = 30 - E;                    // B * 2^e = 2^30: rounding of a product below B stays below 2^31
    const float tscale = ldexpf(1.f, e);
    const double s_fix = ldexp(1.0, -e);    // value of one fixed-point unit

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)bc.x_bytes, 0x00020000);
    const long img = (long)n * H * W * C;
    const int items_step = bc.tr * G.wo;
    const int nsteps = (r_end - r_begin + bc.tr - 1) / bc.tr;
    int base_slot = 0;                               // ring slot of the window's first row
    for (int s = 0; s < nsteps; ++s) {
        const int r_s = r_begin + s * bc.tr;
        const int lo = wlo0 + s * bc.tr * G.sh;       // first row of this step's window
        for (int p0 = 0; p0 < items_step; p0 += bc.ip) {
            const int it = p0 + li;
            const int r = r_s + it / G.wo, wo = it % G.wo;
            // All lanes of an item share `live`, so the item's reductions are whole.
            if (it >= items_step || r >= r_end) continue;
            const long pix = ((long)n * G.ho + r) * G.wo + wo;
            const long item = pix * G.g + g;
            float m[KF ? KF : KMAX_WIN], dm[KF ? KF : KMAX_WIN];
#pragma unroll
            for (int k = 0; k < (KF ? KF : KMAX_WIN); ++k) {
                if (!KF && k >= K) break;
                m[k] = to_f32(mask[item * K + k]);
            }
            if constexpr (SOFTMAX) {
                float mx = m[0];
#pragma unroll
                for (int k = 1; k < (KF ? KF : KMAX_WIN); ++k) {
                    if (!KF && k >= K) break;
                    mx = fmaxf(mx, m[k]);
                }
                float sum = 0.f;
#pragma unroll
                for (int k = 0; k < (KF ? KF : KMAX_WIN); ++k) {
                    if (!KF && k >= K) break;
                    m[k] = exp_nonpos(m[k] - mx);
                    sum += m[k];
                }
                const float inv = 1.0f / sum;
#pragma unroll
                for (int k = 0; k < (KF ? KF : KMAX_WIN); ++k) {
                    if (!KF && k >= K) break;
                    m[k] *= inv;
                }
            }
            float gc[CPL];
            uint32_t gp[RW];
            load_words<RW>(gout + pix * C + (long)g * D + CPL * c4, gp);
            widen<DT, CPL>(gp, gc);
            // Largest |g_c| of this lane's channels; NaN when one of them is
            // NaN (fmaxf would drop it), so that such a lane fails the
            // fixed-point test below.
            float gl = 0.f;
            bool gnan = false;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                gl = fmaxf(gl, fabsf(gc[j]));
                gnan |= gc[j] != gc[j];
            }
            if (gnan) gl = __builtin_nanf("");
            const T* ob = off + item * K * 2;
            const int bx = wo * G.sw - G.pw, by = r * G.sh - G.ph;
            float sdm = 0.f;
            // One tap's channel sums, its writes of grad_offset, and its
            // scatter into grad_x (LDS window or global), given its corners.
            auto tap_finish = [&](int k, float a, float b, int x0, int y0, const uint32_t* o4, const uint32_t* X00,
                                  const uint32_t* X01, const uint32_t* X10, const uint32_t* X11) {
                const float wa = 1.f - a, wb = 1.f - b;
                const float w4[4] = {wa * wb, a * wb, wa * b, a * b};
                // The sample is v_c = sum_q w_q X_qc, linear in the corners, so
                // the channel sums need only each corner's dot product with
                // grad_out, S_q = sum_c g_c X_qc:
                //   sum_c g_c v_c     = sum_q w_q S_q,
                //   sum_c g_c dv_c/da = (1-b)(S01 - S00) + b (S11 - S10),
                //   sum_c g_c dv_c/db = (1-a)(S10 - S00) + a (S11 - S01).
                const float s00 = corner_dot<DT, CPL>(X00, gc, gp), s01 = corner_dot<DT, CPL>(X01, gc, gp);
                const float s10 = corner_dot<DT, CPL>(X10, gc, gp), s11 = corner_dot<DT, CPL>(X11, gc, gp);
                float sm = fmaf(w4[0], s00, fmaf(w4[1], s01, fmaf(w4[2], s10, w4[3] * s11)));
                float sdx = fmaf(wb, s01 - s00, b * (s11 - s10));
                float sdy = fmaf(wa, s10 - s00, a * (s11 - s01));
                if (gx) {
                    const bool small = fabsf(m[k]) * gl < Bf;   // every contribution of this tap below B
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (o4[q] == OOB) continue;   // corner outside the image
                        const int yc = y0 + (q >> 1), xc = x0 + (q & 1);
                        const float mw = m[k] * w4[q];
                        if (fixed && small && yc >= lo && yc < lo + bc.aw) {
                            int slot = base_slot + (yc - lo);
                            slot -= slot >= bc.aw ? bc.aw : 0;
                            unsigned long long* dst = acc + slot * rowe + xc * pstr + CPL * c4;
                            const float mws = mw * tscale;
#pragma unroll
                            for (int j = 0; j < CPL; ++j) atomicAdd(dst + j, to_fixed(mws * gc[j]));
                        } else {
                            float* dst = gx + img + ((long)yc * W + xc) * C + (long)g * D + CPL * c4;
#pragma unroll
                            for (int j = 0; j < CPL; ++j) atomicAdd(dst + j, mw * gc[j]);
                        }
                    }
                }
                // A sample outside the map (all four corners outside) is not
                // read at all: its channel sums are exactly zero, whatever
                // grad_out holds (0 * Inf would otherwise make them NaN).
                if ((o4[0] & o4[1] & o4[2] & o4[3] & OOB) != 0u) sm = sdx = sdy = 0.f;
                sm = lane_sum(sm, lq);
                sdx = lane_sum(sdx, lq);
                sdy = lane_sum(sdy, lq);
                dm[k] = sm;
                sdm += m[k] * sm;
                if (c4 == 0 && goff) {
                    goff[(item * K + k) * 2 + 0] = from_f32<DT>(G.scale * m[k] * sdx);
                    goff[(item * K + k) * 2 + 1] = from_f32<DT>(G.scale * m[k] * sdy);
                }
            };
            if constexpr (KF > 0) {
                // Geometry of every tap first, branch-free: a corner outside the
                // image gets an offset past the end of the buffer (it reads zero
                // and is not scattered); offsets beyond +-2^24 (or not finite)
                // are clamped there, which puts every corner outside.
                const float lim = 16777216.0f;
                uint32_t o4[KF][4];
                float fa[KF], fb[KF];
                int xk[KF], yk[KF];
#pragma unroll
                for (int k = 0; k < KF; ++k) {
                    const int kx = k / KH, ky = k - kx * KH;
                    const float tx = fminf(fmaxf(G.scale * to_f32(ob[2 * k]), -lim), lim);
                    const float ty = fminf(fmaxf(G.scale * to_f32(ob[2 * k + 1]), -lim), lim);
                    const float fx = floorf(tx), fy = floorf(ty);
                    fa[k] = tx - fx;
                    fb[k] = ty - fy;
                    const int x0 = bx + kx * G.dw + (int)fx, y0 = by + ky * G.dh + (int)fy;
                    xk[k] = x0;
                    yk[k] = y0;
                    // A sample exactly on the edge px = -1 (or py = -1) is outside
                    // the map, like any px <= -1: zero value and zero gradient.
                    const bool edge = (x0 == -1 && fa[k] == 0.f) || (y0 == -1 && fb[k] == 0.f);
                    const bool cx0 = (unsigned)x0 < (unsigned)W && !edge, cx1 = (unsigned)(x0 + 1) < (unsigned)W && !edge;
                    const bool cy0 = (unsigned)y0 < (unsigned)H, cy1 = (unsigned)(y0 + 1) < (unsigned)H;
                    const uint32_t b00 = (uint32_t)((img + ((long)y0 * W + x0) * C + (long)g * D + CPL * c4) * ES);
                    const uint32_t bC = (uint32_t)C * ES, bR = (uint32_t)W * C * ES;
                    o4[k][0] = (cy0 && cx0) ? b00 : OOB;
                    o4[k][1] = (cy0 && cx1) ? b00 + bC : OOB;
                    o4[k][2] = (cy1 && cx0) ? b00 + bR : OOB;
                    o4[k][3] = (cy1 && cx1) ? b00 + bR + bC : OOB;
                }
                // The corners of tap k+1 are in flight while tap k is summed.
                uint32_t buf[2][4][RW];
#pragma unroll
                for (int q = 0; q < 4; ++q) load_raw<RW>(xr, o4[0][q], buf[0][q]);
#pragma unroll
                for (int k = 0; k < KF; ++k) {
                    if (k + 1 < KF) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) load_raw<RW>(xr, o4[k + 1][q], buf[(k + 1) & 1][q]);
                    }
                    const uint32_t (*X)[RW] = buf[k & 1];
                    tap_finish(k, fa[k], fb[k], xk[k], yk[k], o4[k], X[0], X[1], X[2], X[3]);
                }
            } else {
#pragma unroll
            for (int k = 0; k < (KF ? KF : KMAX_WIN); ++k) {
                if (!KF && k >= K) break;
                const int kx = k / kh, ky = k - kx * kh;
                const float tx = G.scale * to_f32(ob[2 * k]), ty = G.scale * to_f32(ob[2 * k + 1]);
                float a = 0.f, b = 0.f;
                int x0 = -2, y0 = -2;
                uint32_t o4[4] = {OOB, OOB, OOB, OOB};
                uint32_t X[4][RW];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < RW; ++j) X[q][j] = 0u;
                if (coord_ok(tx) && coord_ok(ty)) {
                    const float fx = floorf(tx), fy = floorf(ty);
                    a = tx - fx;
                    b = ty - fy;
                    x0 = bx + kx * G.dw + (int)fx;
                    y0 = by + ky * G.dh + (int)fy;
                    // px <= -1 or py <= -1 (the edge included), px >= W, py >= H: outside
                    if (x0 >= -1 && x0 < W && y0 >= -1 && y0 < H && !(x0 == -1 && a == 0.f) && !(y0 == -1 && b == 0.f)) {
                        const bool cx0 = x0 >= 0, cx1 = x0 + 1 < W, cy0 = y0 >= 0, cy1 = y0 + 1 < H;
                        const uint32_t b00 = (uint32_t)((img + ((long)y0 * W + x0) * C + (long)g * D + CPL * c4) * ES);
                        const uint32_t bC = (uint32_t)C * ES, bR = (uint32_t)W * C * ES;
                        o4[0] = (cy0 && cx0) ? b00 : OOB;
                        o4[1] = (cy0 && cx1) ? b00 + bC : OOB;
                        o4[2] = (cy1 && cx0) ? b00 + bR : OOB;
                        o4[3] = (cy1 && cx1) ? b00 + bR + bC : OOB;
#pragma unroll
                        for (int q = 0; q < 4; ++q) load_raw<RW>(xr, o4[q], X[q]);
                    }
                }
                tap_finish(k, a, b, x0, y0, o4, X[0], X[1], X[2], X[3]);
            }
            }
            if (c4 == 0 && gmask) {
#pragma unroll
                for (int k = 0; k < (KF ? KF : KMAX_WIN); ++k) {
                    if (!KF && k >= K) break;
                    gmask[item * K + k] = from_f32<DT>(SOFTMAX ? m[k] * (dm[k] - sdm) : dm[k]);
                }
            }
        }
        __syncthreads();
        // Rows that leave the window (all of them after the last step) go to
        // grad_x; their slots are cleared for the rows that enter.
        if (gx) {
            const int nflush = s + 1 < nsteps ? bc.tr * G.sh : bc.aw;
            for (int rr = 0; rr < nflush; ++rr) {
                const int y = lo + rr;
                int slot = base_slot + rr;
                slot -= slot >= bc.aw ? bc.aw : 0;
                unsigned long long* arow = acc + slot * rowe;
                float* grow = gx + img + (long)y * W * C + (long)g * D;
                for (int el = tid; el < W * D; el += nthr) {
                    const int xc = el >> d_log, c = el & (D - 1);
                    const unsigned long long q = arow[xc * pstr + c];
                    if (q != 0ull) {
                        arow[xc * pstr + c] = 0ull;
                        // the 64-bit sum to fp64 (exact below 2^53 units, one rounding
                        // above), scaled exactly, rounded once to fp32
                        const float v = (float)((double)(long long)q * s_fix);
                        atomicAdd(grow + (long)xc * C + c, v);
                    }
                }
            }
            __syncthreads();
        }
        base_slot += bc.tr * G.sh;
        while (base_slot >= bc.aw) base_slot -= bc.aw;
    }
}

}  // namespace

bool plan_bwd_win(const Geom& G, int dtype, const void* x, const void* gout, int lds_limit, int num_cus,
                  BwdWinCfg* bc)
{
    if (G.d % 4 != 0) return false;
    const int nv = G.d % 8 == 0 ? 2 : 1;   // 8 channels per lane when D allows
    const int lq = G.d / (4 * nv);
    if (lq > 64 || (lq & (lq - 1)) != 0) return false;
    if (G.K > KMAX_WIN) return false;
    if ((uintptr_t)x % 16 || (uintptr_t)gout % 16) return false;
    const long x_bytes = (long)G.n * G.h * G.w * G.c * (dtype == DT_F32 ? 4 : 2);
    if (x_bytes >= (1L << 31) - 64) return false;
    int lq_log = 0;
    while ((1 << lq_log) < lq) ++lq_log;
    const int ip_max = 512 / lq;   // items per pass with 512 threads
    int tr, threads;
    if (G.wo <= ip_max) {          // one pass per step of tr output rows
        tr = std::max(1, std::min(ip_max / G.wo, G.ho));
        threads = (tr * G.wo * lq + 63) / 64 * 64;
    } else {                       // one output row per step, several passes
        tr = 1;
        threads = 512;
    }
    const int ipass = threads / lq;
    const long row_bytes = (long)G.w * (G.d + 1) * 8;   // padded pixel stride
    int hy = -1, aw = 0;
    for (int h = 8; h >= 2; --h) {
        const int awh = (tr - 1) * G.sh + (G.kh - 1) * G.dh + 2 * h + 3;
        if ((long)awh * row_bytes + 256 <= lds_limit) {
            hy = h;
            aw = awh;
            break;
        }
    }
    if (hy < 0) return false;
    const long units = (long)G.n * G.g;
    int chunks = (int)std::max(1L, ((long)num_cus + units - 1) / units);
    chunks = std::min(chunks, (G.ho + tr - 1) / tr);
    int chunk_rows = (G.ho + chunks - 1) / chunks;
    chunk_rows = (chunk_rows + tr - 1) / tr * tr;
    chunks = (G.ho + chunk_rows - 1) / chunk_rows;
    if (units * chunks >= (1L << 31)) return false;
    bc->lq_log = lq_log;
    bc->nv = nv;
    bc->ip = ipass;
    bc->tr = tr;
    bc->hy = hy;
    bc->aw = aw;
    bc->chunk_rows = chunk_rows;
    bc->chunks = chunks;
    bc->nwg = (int)(units * chunks);
    bc->threads = threads;
    bc->lds_bytes = (int)(aw * row_bytes);
    bc->x_bytes = (uint32_t)x_bytes;
    return true;
}

namespace {

template <int DT>
hipError_t launch_win_typed(const Geom& G, const BwdWinCfg& bc, const void* x, const void* off, const void* mask,
                            const void* gout, float* gx, void* goff, void* gmask, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const dim3 grid(bc.nwg), block(bc.threads);
#define DCN_BWIN(KHV, KWV, SM)                                                                                   \
    {                                                                                                           \
        auto* fn = bc.nv == 2 ? dcn_bwd_win<DT, KHV, KWV, SM, 2> : dcn_bwd_win<DT, KHV, KWV, SM, 1>;            \
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,          \
                                           bc.lds_bytes);                                                       \
        if (e != hipSuccess) return e;                                                                          \
        fn<<<grid, block, bc.lds_bytes, s>>>(G, bc, (const T*)x, (const T*)off, (const T*)mask, (const T*)gout,  \
                                             gx, (T*)goff, (T*)gmask);                                           \
    }
    const bool k33 = G.kh == 3 && G.kw == 3;
    if (k33 && G.softmax) DCN_BWIN(3, 3, true)
    else if (k33) DCN_BWIN(3, 3, false)
    else if (G.softmax) DCN_BWIN(0, 0, true)
    else DCN_BWIN(0, 0, false)
#undef DCN_BWIN
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_backward_win(const Geom& G, const BwdWinCfg& bc, int dtype, const void* x, const void* off,
                                   const void* mask, const void* gout, float* gx, void* goff, void* gmask,
                                   hipStream_t s)
{
    switch (dtype) {
        case DT_F32: return launch_win_typed<DT_F32>(G, bc, x, off, mask, gout, gx, goff, gmask, s);
        case DT_F16: return launch_win_typed<DT_F16>(G, bc, x, off, mask, gout, gx, goff, gmask, s);
        case DT_BF16: return launch_win_typed<DT_BF16>(G, bc, x, off, mask, gout, gx, goff, gmask, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
