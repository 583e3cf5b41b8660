// DCN forward, LDS sliding-window kernel for gfx950.
//
// Same operator as dcn_forward.hip ("DCNv4: Unbounded Weights", "Why Is
// Sampling Just 9 Points Still Slow?": y_g(p0) = sum_k m_gk x_g(p0 + p_k +
// dp_gk), bilinear reads with zero outside the map per "InternImage:
// Deformable Convolutions at Scale", Ch.2; softmax over K for DCNv3, Ch.3).
//
// Why a different kernel: on gfx950 a scattered 16-32 byte read through the
// vector L1 costs about one cache-line lookup (~2.3 clocks per line per CU),
// so gathering 36 corners per output from L1 runs far below HBM speed; the
// LDS serves random 16-byte reads several times faster.  Each workgroup
// therefore owns one image, a set of GS channel groups and a chunk of output
// rows.  It keeps a ring of input rows of those groups in LDS (two zero
// columns on the left, one on the right, plus a mirror of slot 0 after the
// last slot so the row below any slot is the next slot in memory) and walks
// down the chunk TR output rows per step:
//   - the rows a step may read through LDS form the window [lo, lo + NW): the
//     3x3 footprint of its output rows plus HY halo rows above and below for
//     the learned offsets;
//   - while a step computes, buffer-to-LDS loads bring in the rows the next
//     step adds, with no VGPR round trip, and each lane loads the offsets
//     and mask of its next item into registers (no LDS staging area, so the
//     whole LDS goes to the ring);
//   - a sample whose two rows fall outside the window (|dy| > HY) is given
//     zero weight in the LDS pass and read with global loads in a tail pass by
//     the lanes that need it;
//   - a tap that reads nothing through LDS (outside the map, or in the tail)
//     points at LDS address 0, the two left-hand zero columns of slots 0
//     and 1, so its four corners read zeros: a zero weight times a
//     non-finite x elsewhere would otherwise turn the sum into NaN.
// Lane = one (output pixel, group) item holding all D channels: the tap
// geometry is computed once per item and reused for every channel; fp32
// accumulation; 16-byte vector stores, one writer per output element.  A
// group wider than 32 bytes per pixel runs as several items of 32 bytes that
// share the group's offsets and mask (the plan's split_log).
// WMAX is the workgroup's wave count bound: 16 (four waves per SIMD, <=128
// VGPRs), the next tap's geometry computed while its reads land; 8 where a
// 1024-thread plan does not fit, with the geometry of all taps computed
// first and the next tap's reads in flight during the math.
#include "dcn_device.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr uint32_t OOB = 0x80000000u;   // buffer offset past any accepted tensor: reads as zero
constexpr int ROW_IT = 4;               // per-thread 16-byte chunks of one input row

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ u32x4 lds_ld16(const unsigned char* base, uint32_t off)
{
    return *reinterpret_cast<const u32x4*>(base + off);
}

// acc[0..V) += w * (16 bytes of x in the storage type)
template <int DT>
__device__ __forceinline__ void fma16(float* acc, float w, u32x4 r)
{
    const uint32_t q[4] = {r.x, r.y, r.z, r.w};
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, __uint_as_float(q[i]), acc[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DT_F16) {
                acc[2 * i] = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i] & 0xffffu)), acc[2 * i]);
                acc[2 * i + 1] = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i] >> 16)), acc[2 * i + 1]);
            } else {
                acc[2 * i] = fmaf(w, __uint_as_float(q[i] << 16), acc[2 * i]);
                acc[2 * i + 1] = fmaf(w, __uint_as_float(q[i] & 0xffff0000u), acc[2 * i + 1]);
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ float h2f(uint32_t h16)
{
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
    return __uint_as_float(h16 << 16);
}

template <int DT, int KH, int KW, bool SOFTMAX, int NCH, int WMAX>
__global__ __launch_bounds__(WMAX * 64) __attribute__((amdgpu_waves_per_eu(WMAX / 4, WMAX / 4))) void dcn_fwd_ring(
    Geom G, RingCfg rc, const typename Elem<DT>::T* __restrict__ x, const typename Elem<DT>::T* __restrict__ off,
    const typename Elem<DT>::T* __restrict__ mask, typename Elem<DT>::T* __restrict__ out)
{
    using T = typename Elem<DT>::T;
    constexpr int ES = sizeof(T);
    constexpr int V = 16 / ES;               // channels per 16-byte chunk
    constexpr int KF = KH * KW;
    constexpr uint32_t K2B = KF * 2 * ES;    // offset bytes of one item
    constexpr uint32_t KMB = KF * ES;        // mask bytes of one item
    static_assert(KF > 0, "ring kernel is instantiated for fixed kernels");
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* ring = lds;

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    int L = blockIdx.x;
    if (rc.nwg % 8 == 0) L = (blockIdx.x % 8) * (rc.nwg / 8) + blockIdx.x / 8;   // neighbours share an XCD
    const int chunk = L % rc.chunks;
    const int ng = L / rc.chunks;
    const int gset = ng % rc.gsets, n = ng / rc.gsets;
    const int g0 = gset * rc.gs;
    const int r_begin = chunk * rc.chunk_rows;
    const int r_end = min(G.ho, r_begin + rc.chunk_rows);
    if (r_begin >= r_end) return;
    const int nsteps = (r_end - r_begin + rc.tr - 1) / rc.tr;
    const int adv = rc.tr * G.sh;                       // window advance per step (input rows)
    const int lo0 = r_begin * G.sh - G.ph - rc.hy;      // first row of the first window

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)rc.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc((void*)off, (short)0, (int)rc.off_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc((void*)mask, (short)0, (int)rc.mask_bytes, 0x00020000);
    const uint32_t pix_g = (uint32_t)G.c * ES;          // global bytes per pixel
    const uint32_t row_bytes = (uint32_t)G.w * pix_g;
    const uint32_t img_bytes = (uint32_t)G.h * row_bytes;
    const uint32_t gsize = (uint32_t)G.d * ES;
    const uint32_t goff = (uint32_t)g0 * gsize;         // first byte of the group set in a global pixel

    // Per-lane source offsets of the 16-byte chunks this lane copies in every
    // input row (the same chunks for every row).
    const uint32_t row_chunks = (uint32_t)G.w * rc.cpp;
    uint32_t row_src[ROW_IT];
#pragma unroll
    for (int i = 0; i < ROW_IT; ++i) {
        const uint32_t t = (uint32_t)(wave + i * nwaves) * 64u + lane;
        const uint32_t pix = t / rc.cpp, u = t - pix * rc.cpp;
        row_src[i] = t < row_chunks ? pix * pix_g + goff + 16u * u : OOB;
    }
    auto load_row = [&](int row) {
        const int slot = (row - lo0) % rc.R;
        const bool inside = (unsigned)row < (unsigned)G.h;
        const uint32_t base = n * img_bytes + (uint32_t)row * row_bytes;
#pragma unroll
        for (int i = 0; i < ROW_IT; ++i) {
            if (i >= rc.row_iters) break;
            const uint32_t c = (uint32_t)(wave + i * nwaves) * 1024u;
            if (row_src[i] != OOB) {
                const uint32_t src = inside ? base + row_src[i] : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(ring + slot * rc.pitch + 2 * rc.pb + c), 16,
                                                         src, 0, 0, 0);
                if (slot == 0)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(ring + rc.R * rc.pitch + 2 * rc.pb + c),
                                                             16, src, 0, 0, 0);
            }
        }
    };

    // This lane's item within every step: row rl of the step, column c, group gl of the set.
    const int items_row = G.wo * rc.gs;
    const int rl = tid / items_row;
    const int rem = tid - rl * items_row;
    const int c = rem / rc.gs, gl = rem - c * rc.gs;
    const int g = g0 + gl;

    // Offsets and mask of this lane's item in a step, loaded into registers
    // one step ahead (no LDS staging, so the whole LDS goes to the ring):
    // the item's KF offset pairs and the dwords that hold its KF modulation
    // scalars.  16-bit scalars form a run that starts at byte 0 or 2 of its
    // first dword, re-aligned with a funnel shift.
    constexpr int OW = (int)(K2B / 4);            // offset dwords per item
    constexpr int MW = ES == 4 ? KF : KF / 2 + 1; // mask dwords loaded per item
    uint32_t po[OW], pmr[MW], psh = 0;
    auto load_offsets = [&](int s) {
        const int rr = r_begin + s * rc.tr + rl;
        const bool v = rl < rc.tr && rr < r_end;
        const uint32_t item = ((uint32_t)(n * G.ho + rr) * G.wo + c) * (G.g >> rc.split_log) + (g >> rc.split_log);
        const uint32_t ob = v ? item * K2B : OOB;
        const uint32_t mb = v ? (item * KMB) & ~3u : OOB;
        psh = ((item * KMB) & 3u) * 8u;
#pragma unroll
        for (int i = 0; i < OW; i += 4) {
            if (i + 4 <= OW) {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(orr, ob + 4u * i, 0, 0);
                po[i] = a.x; po[i + 1] = a.y; po[i + 2] = a.z; po[i + 3] = a.w;
            } else {
#pragma unroll
                for (int j = i; j < OW; ++j) po[j] = __builtin_amdgcn_raw_buffer_load_b32(orr, ob + 4u * j, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < MW; i += 4) {
            if (i + 4 <= MW) {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(mr, mb + 4u * i, 0, 0);
                pmr[i] = a.x; pmr[i + 1] = a.y; pmr[i + 2] = a.z; pmr[i + 3] = a.w;
            } else {
#pragma unroll
                for (int j = i; j < MW; ++j) pmr[j] = __builtin_amdgcn_raw_buffer_load_b32(mr, mb + 4u * j, 0, 0);
            }
        }
    };

    // Zero the border columns of every ring slot, mirror included (never
    // written again): LDS columns 0, 1 (image columns -2, -1) and W+2 (image
    // column W).
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < (rc.R + 1) * 3 * rc.cpp; i += nthr) {
            const int slot = i / (3 * rc.cpp), j = i - slot * 3 * rc.cpp;
            const uint32_t col_off = j < 2 * rc.cpp ? 16u * j : (uint32_t)(G.w + 2) * rc.pb + 16u * (j - 2 * rc.cpp);
            *reinterpret_cast<u32x4*>(ring + slot * rc.pitch + col_off) = z;
        }
    }
    for (int rr = 0; rr < rc.nw; ++rr) load_row(lo0 + rr);
    load_offsets(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Byte offset of this lane's group within LDS column 1 (image column -1):
    // a tap's left corners sit at column xs + 1 for xs = x0 + 1.
    const uint32_t gbyte = (uint32_t)gl * gsize + (uint32_t)rc.pb;
    const float lim = 16777216.0f;
    // Window-relative row and LDS column of each tap's top-left corner before
    // the offset (they do not change from step to step): bx0 + kx*dw and
    // by0 + ky*dh, the second term uniform.  16-bit offsets take them as
    // floats, one register per tap (the multiply-add that forms a position
    // adds them); fp32 adds them as integers, two registers in all.
    const int bx0 = c * G.sw - G.pw + 1;
    const int by0 = (r_begin + rl) * G.sh - G.ph - lo0;
    float bxf[ES == 2 ? KW : 1], byf[ES == 2 ? KH : 1];
    if constexpr (ES == 2) {
#pragma unroll
        for (int kx = 0; kx < KW; ++kx) bxf[kx] = (float)(bx0 + kx * G.dw);
#pragma unroll
        for (int ky = 0; ky < KH; ++ky) byf[ky] = (float)(by0 + ky * G.dh);
    }

    for (int s = 0; s < nsteps; ++s) {
        const int r_s = r_begin + s * rc.tr;
        const int r = r_s + rl;
        const bool live = rl < rc.tr && r < r_end;
        const int lo = lo0 + s * adv;
        const int slot_lo = (s * adv) % rc.R;

        // ---- offsets and mask of this lane's item, then the next step's loads.
        // 16-bit offset pairs stay packed (pc) until a tap's geometry needs
        // them, which keeps 9 registers free while the next step's loads are
        // in flight.
        float dx[KF], dy[KF], m[KF];
        uint32_t pc[KF];
        if constexpr (ES == 4) {
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                dx[k] = __uint_as_float(po[2 * k]);
                dy[k] = __uint_as_float(po[2 * k + 1]);
                m[k] = __uint_as_float(pmr[k]);
            }
        } else {
            uint32_t mw[MW];
#pragma unroll
            for (int i = 0; i < MW; ++i) mw[i] = __builtin_amdgcn_alignbit(i + 1 < MW ? pmr[i + 1] : 0u, pmr[i], psh);
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                pc[k] = po[k];
                m[k] = h2f<DT>((k & 1) ? mw[k >> 1] >> 16 : mw[k >> 1] & 0xffffu);
            }
        }

        // ---- the next step's new rows go straight to LDS, its offsets to
        // registers (fp32 in 1024-thread workgroups: piece by piece as the
        // taps consume them, below)
        constexpr bool TAPWISE = ES == 4 && WMAX == 16;
        if (s + 1 < nsteps) {
            if constexpr (!TAPWISE) load_offsets(s + 1);
            for (int rr = 0; rr < adv; ++rr) load_row(lo + rc.nw + rr);
        }

        if (live) {
            float smax = 0.f, sinv = 1.f;   // softmax max and 1/sum, kept for the tail
            if constexpr (SOFTMAX) {
                float mx = m[0];
#pragma unroll
                for (int k = 1; k < KF; ++k) mx = fmaxf(mx, m[k]);
                float sum = 0.f;
#pragma unroll
                for (int k = 0; k < KF; ++k) { m[k] = exp_nonpos(m[k] - mx); sum += m[k]; }
                const float inv = 1.0f / sum;
#pragma unroll
                for (int k = 0; k < KF; ++k) m[k] *= inv;
                smax = mx;
                sinv = inv;
            }
            float acc[NCH * V];
#pragma unroll
            for (int q = 0; q < NCH * V; ++q) acc[q] = 0.f;
            const uint32_t o01 = (uint32_t)rc.pb, o10 = (uint32_t)rc.pitch, o11 = (uint32_t)(rc.pitch + rc.pb);
            uint32_t fb = 0;
            // Tap k's geometry: the LDS address of its top-left corner (the
            // others are +pb, +pitch, +pitch+pb) and its four weights.
            auto geo = [&](int k, uint32_t& Ak, float& w00, float& w01, float& w10, float& w11) {
                const int kx = k / KH, ky = k - (k / KH) * KH;
                float dxk, dyk;
                if constexpr (ES == 4) {
                    dxk = dx[k];
                    dyk = dy[k];
                } else {
                    dxk = h2f<DT>(pc[k] & 0xffffu);
                    dyk = h2f<DT>(pc[k] >> 16);
                }
                int xs, yi;   // x0 + 1 (LDS column of the left corners - 1), window row of the top corners
                float a, b;   // fractions
                if constexpr (ES == 2) {
                    // 16-bit offsets: the position sigma*d + base in one
                    // multiply-add (v_fma_mix_f32 takes the 16-bit operand),
                    // then floor-and-convert and the fraction in one
                    // instruction each; the compiler forms neither
                    // v_cvt_flr_i32_f32 nor the fused base, hence the asm.
                    // The sum rounds to fp32 (at most 2^-24 of |position|),
                    // which moves the bilinear sample continuously by that
                    // much, far below the 16-bit output's rounding.
                    const float tx = fminf(fmaxf(fmaf(G.scale, dxk, bxf[kx]), -lim), lim);
                    const float ty = fminf(fmaxf(fmaf(G.scale, dyk, byf[ky]), -lim), lim);
                    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(xs) : "v"(tx));
                    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(yi) : "v"(ty));
                    a = __builtin_amdgcn_fractf(tx);
                    b = __builtin_amdgcn_fractf(ty);
                } else {
                    // fp32: floor and fraction of sigma*d alone, then the
                    // integer base, so the fraction is exact.
                    const float tx = fminf(fmaxf(G.scale * dxk, -lim), lim);
                    const float ty = fminf(fmaxf(G.scale * dyk, -lim), lim);
                    const float fx = floorf(tx), fy = floorf(ty);
                    a = tx - fx;
                    b = ty - fy;
                    xs = bx0 + kx * G.dw + (int)fx;
                    yi = by0 + ky * G.dh + (int)fy;
                }
                const bool colok = (unsigned)xs <= (unsigned)G.w;   // image column in [-1, W-1]
                const bool inwin = (unsigned)yi < (unsigned)(rc.nw - 1);
                fb |= (colok && !inwin) ? (1u << k) : 0u;
                const bool use = colok && inwin;
                uint32_t s0 = (uint32_t)(slot_lo + yi);
                s0 = min(s0, s0 - (uint32_t)rc.R);                  // wrap once
                const uint32_t addr = __umul24(s0, (uint32_t)rc.pitch) + __umul24((uint32_t)xs, (uint32_t)rc.pb) + gbyte;
                Ak = use ? addr : 0u;   // LDS columns 0, 1 of slots 0, 1: zeros
                const float mm = use ? m[k] : 0.f;
                // m(1-a) = m - m*a, m(1-a)(1-b) = m(1-a) - m(1-a)b, ...: one
                // multiply per pair of weights
                const float mb = mm * a, ma = mm - mb;
                w10 = ma * b;
                w00 = ma - w10;
                w11 = mb * b;
                w01 = mb - w11;
            };
            // The four corners' addresses are pointers into the ring, so that
            // the 16-byte chunk offsets fold into the reads' immediate offsets.
            auto issue = [&](uint32_t Ak, u32x4* d) {
                const unsigned char* p00 = ring + Ak;
                const unsigned char* p01 = p00 + o01;
                const unsigned char* p10 = p00 + o10;
                const unsigned char* p11 = p00 + o11;
#pragma unroll
                for (int q = 0; q < NCH; ++q) {
                    d[4 * q + 0] = *reinterpret_cast<const u32x4*>(p00 + 16 * q);
                    d[4 * q + 1] = *reinterpret_cast<const u32x4*>(p01 + 16 * q);
                    d[4 * q + 2] = *reinterpret_cast<const u32x4*>(p10 + 16 * q);
                    d[4 * q + 3] = *reinterpret_cast<const u32x4*>(p11 + 16 * q);
                }
            };
            if constexpr (WMAX == 16) {
                // Four waves per SIMD hide the LDS latency, so registers go to
                // occupancy: one tap's data in flight, the next tap's geometry
                // computed while it lands.
                //
                // fp32 offsets and mask take 27 registers per item: rather
                // than hold the next step's set beside this one, the registers
                // are refilled with the next step's values as soon as the taps
                // that read them are done, in the same 16-byte pieces as a
                // whole-set load (offset dwords 4i..4i+3 after tap 2i+1, mask
                // dwords 4j..4j+3 after tap 4j+3, the rest after the last
                // tap).  A lane live in the next step is live in this one (its
                // row only moves down), so only live lanes load.
                uint32_t nob = OOB, nmb = OOB;
                if constexpr (TAPWISE) {
                    const int rr = r + rc.tr;
                    if (s + 1 < nsteps && rr < r_end) {
                        const uint32_t item =
                            ((uint32_t)(n * G.ho + rr) * G.wo + c) * (G.g >> rc.split_log) + (g >> rc.split_log);
                        nob = item * K2B;
                        nmb = item * KMB;
                    }
                }
                auto refill = [&](int k) {
                    if constexpr (TAPWISE) {
                        // offset dwords [4i, 4i + 4) once tap k has read dword 2k + 1
#pragma unroll
                        for (int i = 0; i < OW; i += 4) {
                            const int last = i + 4 <= OW ? (i + 3) / 2 : KF - 1;
                            if (k != last) continue;
                            if (i + 4 <= OW) {
                                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(orr, nob + 4u * i, 0, 0);
                                po[i] = v.x; po[i + 1] = v.y; po[i + 2] = v.z; po[i + 3] = v.w;
                            } else {
#pragma unroll
                                for (int j = i; j < OW; ++j) po[j] = __builtin_amdgcn_raw_buffer_load_b32(orr, nob + 4u * j, 0, 0);
                            }
                        }
                        // mask dwords [4i, 4i + 4) once tap k has read dword k
#pragma unroll
                        for (int i = 0; i < MW; i += 4) {
                            const int last = i + 4 <= MW ? i + 3 : KF - 1;
                            if (k != last) continue;
                            if (i + 4 <= MW) {
                                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(mr, nmb + 4u * i, 0, 0);
                                pmr[i] = v.x; pmr[i + 1] = v.y; pmr[i + 2] = v.z; pmr[i + 3] = v.w;
                            } else {
#pragma unroll
                                for (int j = i; j < MW; ++j) pmr[j] = __builtin_amdgcn_raw_buffer_load_b32(mr, nmb + 4u * j, 0, 0);
                            }
                        }
                    }
                };
                uint32_t Ac;
                float c00, c01, c10, c11;
                geo(0, Ac, c00, c01, c10, c11);
                refill(0);
                u32x4 cur[4 * NCH];
                issue(Ac, cur);
#pragma unroll
                for (int k = 0; k < KF; ++k) {
                    uint32_t An = 0;
                    float n00 = 0.f, n01 = 0.f, n10 = 0.f, n11 = 0.f;
                    if (k + 1 < KF) {
                        geo(k + 1, An, n00, n01, n10, n11);
                        refill(k + 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // A wave whose tap data has landed goes first on its SIMD
                    // while it multiplies (wave priority, not a stream
                    // priority): the others' reads then wait in the LDS queue
                    // behind math rather than the math behind them (stage-1
                    // f16 45.2 -> 43.4 us, stage-2 25.5 -> 24.4 us).
                    __builtin_amdgcn_s_setprio(2);
#pragma unroll
                    for (int q = 0; q < NCH; ++q) {
                        fma16<DT>(acc + q * V, c00, cur[4 * q + 0]);
                        fma16<DT>(acc + q * V, c01, cur[4 * q + 1]);
                        fma16<DT>(acc + q * V, c10, cur[4 * q + 2]);
                        fma16<DT>(acc + q * V, c11, cur[4 * q + 3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(0);
                    if (k + 1 < KF) {
                        issue(An, cur);
                        c00 = n00; c01 = n01; c10 = n10; c11 = n11;
                    }
                }
            } else {
                // Geometry of all taps first: the LDS address of the top-left
                // corner (the others are +pb, +pitch, +pitch+pb) and four weights.
                uint32_t A[KF];
                float W00[KF], W01[KF], W10[KF], W11[KF];
#pragma unroll
                for (int k = 0; k < KF; ++k) geo(k, A[k], W00[k], W01[k], W10[k], W11[k]);
                // Reads of tap k+1 are in flight while tap k accumulates.  Chunk q
                // of a corner sits 16*q bytes past its first, an immediate offset
                // of the read.  (Rotating the chunk order between neighbouring
                // lanes spreads a read over more LDS bank groups, but its address
                // arithmetic cost more than the conflicts it saved.)
                u32x4 cur[4 * NCH], nxt[4 * NCH];
                issue(A[0], cur);
#pragma unroll
                for (int k = 0; k < KF; ++k) {
                    if (k + 1 < KF) issue(A[k + 1], nxt);
                    __builtin_amdgcn_sched_barrier(0);   // keep the next tap's reads ahead of this tap's math
#pragma unroll
                    for (int q = 0; q < NCH; ++q) {
                        fma16<DT>(acc + q * V, W00[k], cur[4 * q + 0]);
                        fma16<DT>(acc + q * V, W01[k], cur[4 * q + 1]);
                        fma16<DT>(acc + q * V, W10[k], cur[4 * q + 2]);
                        fma16<DT>(acc + q * V, W11[k], cur[4 * q + 3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (k + 1 < KF) {
#pragma unroll
                        for (int q = 0; q < 4 * NCH; ++q) cur[q] = nxt[q];
                    }
                }
            }
            // Tail: samples outside the window that may touch the image, read
            // from global memory.  Each lane walks only its own such taps, so a
            // wave runs as many iterations as its busiest lane; the tap's
            // offsets and modulation are read again from global memory rather
            // than indexed in registers (a dynamic index into the prefetched
            // registers would move them to scratch).
            if (fb) {
                const uint32_t base_img = n * img_bytes + (uint32_t)g * gsize;
                const uint32_t item = ((uint32_t)(n * G.ho + r) * G.wo + c) * (G.g >> rc.split_log) + (g >> rc.split_log);
                while (fb) {
                    const int k = __builtin_ctz(fb);
                    fb &= fb - 1u;
                    const int kx = k / KH, ky = k - kx * KH;
                    float dxk, dyk, mk;
                    if constexpr (ES == 4) {
                        const uint32_t o = item * K2B + 8u * k;
                        dxk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orr, o, 0, 0));
                        dyk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orr, o + 4u, 0, 0));
                        mk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, item * KMB + 4u * k, 0, 0));
                    } else {
                        const uint32_t pr = __builtin_amdgcn_raw_buffer_load_b32(orr, item * K2B + 4u * k, 0, 0);
                        dxk = h2f<DT>(pr & 0xffffu);
                        dyk = h2f<DT>(pr >> 16);
                        mk = h2f<DT>(__builtin_amdgcn_raw_buffer_load_b16(mr, item * KMB + 2u * k, 0, 0));
                    }
                    if constexpr (SOFTMAX) mk = exp_nonpos(mk - smax) * sinv;
                    const float tx = fminf(fmaxf(G.scale * dxk, -lim), lim);
                    const float ty = fminf(fmaxf(G.scale * dyk, -lim), lim);
                    const float fx = floorf(tx), fy = floorf(ty);
                    const float a = tx - fx, b = ty - fy;
                    const int x0 = c * G.sw - G.pw + kx * G.dw + (int)fx;
                    const int y0 = (r_begin + rl) * G.sh - G.ph + ky * G.dh + (int)fy + s * adv;
                    const bool cx0 = (unsigned)x0 < (unsigned)G.w, cx1 = (unsigned)(x0 + 1) < (unsigned)G.w;
                    const bool cy0 = (unsigned)y0 < (unsigned)G.h, cy1 = (unsigned)(y0 + 1) < (unsigned)G.h;
                    const uint32_t p00 = base_img + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_g;
                    const uint32_t o00 = (cy0 && cx0) ? p00 : OOB, o01g = (cy0 && cx1) ? p00 + pix_g : OOB;
                    const uint32_t o10g = (cy1 && cx0) ? p00 + row_bytes : OOB;
                    const uint32_t o11g = (cy1 && cx1) ? p00 + row_bytes + pix_g : OOB;
                    const float ma = mk * (1.f - a), mb = mk * a;
#pragma unroll
                    for (int q = 0; q < NCH; ++q) {
                        const uint32_t qo = 16u * q;
                        fma16<DT>(acc + q * V, ma * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o00 + qo, 0, 0));
                        fma16<DT>(acc + q * V, mb * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o01g + qo, 0, 0));
                        fma16<DT>(acc + q * V, ma * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o10g + qo, 0, 0));
                        fma16<DT>(acc + q * V, mb * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o11g + qo, 0, 0));
                    }
                }
            }
            T* op = out + (((long)(n * G.ho + r) * G.wo + c) * G.c + (long)g * G.d);
#pragma unroll
            for (int q = 0; q < NCH; ++q) store_vec<DT>(op + q * V, acc + q * V);
        }

        __builtin_amdgcn_s_waitcnt(0);   // this wave's buffer-to-LDS loads have landed
        __syncthreads();
    }
}

template <int DT, bool SOFTMAX, int NCHV, int WM>
hipError_t launch_one(const Geom& G, const RingCfg& rc, const void* x, const void* off, const void* mask, void* out,
                      hipStream_t s)
{
    using T = typename Elem<DT>::T;
    auto* fn = dcn_fwd_ring<DT, 3, 3, SOFTMAX, NCHV, WM>;
    const hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, rc.lds_bytes);
    if (e != hipSuccess) return e;
    fn<<<dim3(rc.nwg), dim3(rc.threads), rc.lds_bytes, s>>>(G, rc, (const T*)x, (const T*)off, (const T*)mask,
                                                             (T*)out);
    return hipGetLastError();
}

template <int DT, bool SOFTMAX>
hipError_t launch_ring_typed(const Geom& G, const RingCfg& rc, const void* x, const void* off, const void* mask,
                             void* out, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const int nch = G.d * (int)sizeof(T) / 16;   // 1 or 2: lane items are at most 32 bytes
    const bool wide = rc.wmax == 16;
    if (wide && nch == 1) return launch_one<DT, SOFTMAX, 1, 16>(G, rc, x, off, mask, out, s);
    if (wide && nch == 2) return launch_one<DT, SOFTMAX, 2, 16>(G, rc, x, off, mask, out, s);
    if (wide) return hipErrorInvalidValue;
    switch (nch) {
        case 1: return launch_one<DT, SOFTMAX, 1, 8>(G, rc, x, off, mask, out, s);
        case 2: return launch_one<DT, SOFTMAX, 2, 8>(G, rc, x, off, mask, out, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dcn_forward_ring(const Geom& G, const RingCfg& rc, int dtype, const void* x, const void* off,
                                   const void* mask, void* out, hipStream_t s)
{
    switch (dtype * 2 + (G.softmax ? 1 : 0)) {
        case DT_F32 * 2 + 0: return launch_ring_typed<DT_F32, false>(G, rc, x, off, mask, out, s);
        case DT_F32 * 2 + 1: return launch_ring_typed<DT_F32, true>(G, rc, x, off, mask, out, s);
        case DT_F16 * 2 + 0: return launch_ring_typed<DT_F16, false>(G, rc, x, off, mask, out, s);
        case DT_F16 * 2 + 1: return launch_ring_typed<DT_F16, true>(G, rc, x, off, mask, out, s);
        case DT_BF16 * 2 + 0: return launch_ring_typed<DT_BF16, false>(G, rc, x, off, mask, out, s);
        case DT_BF16 * 2 + 1: return launch_ring_typed<DT_BF16, true>(G, rc, x, off, mask, out, s);
    }
    return hipErrorInvalidValue;
}

// Choose the group set, rows per step, halo and chunking for geometry G, or
// return false when the sliding-window kernel does not apply.
bool plan_ring(const Geom& G0, int dtype, const void* x, const void* off, const void* mask, const void* out,
               int lds_limit, int num_cus, RingCfg* rc, Geom* gk)
{
    if (G0.kh != 3 || G0.kw != 3) return false;
    const int es = dtype == DT_F32 ? 4 : 2;
    if (G0.d * es % 16 != 0) return false;
    if ((uintptr_t)x % 16 || (uintptr_t)off % 16 || (uintptr_t)mask % 16 || (uintptr_t)out % 16) return false;
    const long x_bytes = (long)G0.n * G0.h * G0.w * G0.c * es;
    const long off_bytes = (long)G0.items * G0.K * 2 * es, mask_bytes = (long)G0.items * G0.K * es;
    if (x_bytes >= (1L << 31) || off_bytes >= (1L << 31) - 64 || mask_bytes >= (1L << 31) - 64) return false;
    // A group wider than lane_bytes per pixel runs as 2^split_log groups of
    // lane_bytes, each lane item with its own share of the channels and the
    // group's offsets and mask: the tap geometry is then computed once per
    // lane item, but a lane's sums and corner data stay within the registers
    // of the 1024-thread 2-chunk kernel.  At 56x56x128 with 4 groups of 32
    // channels: f16 71 us against 75 for 64-byte items in 512-thread groups;
    // f32 102 us against 117 for 64-byte items; 56x56x64 f32 (16 channels a
    // group): 66 us against 72.
    const int lane_bytes = 32;
    int split_log = 0;
    while ((G0.d * es >> split_log) > lane_bytes) ++split_log;
    if (split_log > 0 && (G0.d % (1 << split_log) != 0 || (G0.d >> split_log) * es != lane_bytes)) return false;
    Geom G = G0;
    G.g = G0.g << split_log;
    G.d = G0.d >> split_log;
    G.items = G0.items << split_log;
    if ((long)G0.items << split_log >= (1L << 31)) return false;
    const int nch = G.d * es / 16;
    if (nch != 1 && nch != 2) return false;
    *gk = G;
    rc->split_log = split_log;

    const int HY_MIN = 4, HY_MAX = 8;
    // The plan for gs groups per workgroup and tr output rows per step, if
    // its ring fits in `lds` bytes with a halo of at least HY_MIN rows: cus is
    // the number of workgroups wanted at least (CUs times workgroups per CU),
    // wmax the kernel variant.
    auto fit = [&](int gs, int tr, int max_thr, long cus, long lds, int wmax) -> bool {
        const int items_row = G.wo * gs;
        const int items_step = tr * items_row;
        const int threads = (items_step + 63) / 64 * 64;
        const int pb = gs * G.d * es;
        const int cpp = pb / 16;
        // W image columns, two zero columns left and one right, and 5 bank
        // groups of skew so that nearby rows spread over the banks.
        const long pitch = (long)(G.w + 3) * pb + 80;
        const int nwaves = threads / 64;
        const int row_iters = (int)((((long)G.w * cpp + 63) / 64 + nwaves - 1) / nwaves);
        if (row_iters > 4 || threads > max_thr) return false;   // ROW_IT
        const int adv = tr * G.sh;
        int hy = -1, nw = 0, R = 0;
        for (int h = HY_MAX; h >= HY_MIN; --h) {
            const int nwh = (tr - 1) * G.sh + (G.kh - 1) * G.dh + 2 + 2 * h;
            const int Rh = nwh + adv;
            if ((long)(Rh + 1) * pitch <= lds) {
                hy = h;
                nw = nwh;
                R = Rh;
                break;
            }
        }
        if (hy < 0) return false;
        const int gsets = G.g / gs;
        const long units = (long)G.n * gsets;
        int chunks = (int)std::max(1L, (cus + units - 1) / units);
        chunks = std::min(chunks, (G.ho + tr - 1) / tr);
        int chunk_rows = (G.ho + chunks - 1) / chunks;
        // A chunk need not be a whole number of steps (its last step may be
        // partial): rounding it up would leave the last chunk short.
        chunks = (G.ho + chunk_rows - 1) / chunk_rows;
        if (units * chunks >= (1L << 31)) return false;
        rc->gs = gs;
        rc->gsets = gsets;
        rc->pb = pb;
        rc->cpp = cpp;
        rc->pitch = (int)pitch;
        rc->R = R;
        rc->nw = nw;
        rc->hy = hy;
        rc->tr = tr;
        rc->chunk_rows = chunk_rows;
        rc->chunks = chunks;
        rc->nwg = (int)(units * chunks);
        rc->threads = threads;
        rc->wmax = wmax;
        rc->row_iters = row_iters;
        rc->ring_bytes = (int)((R + 1) * pitch);
        rc->lds_bytes = rc->ring_bytes;   // offsets and mask go to registers, not LDS
        // Buffer loads range-check each dword: a dword that straddles num_records
        // reads as zero.  Rounding the extents up to whole dwords keeps the last
        // values of an odd-length 16-bit tensor readable; the extra bytes share
        // a dword (and so a page) with valid data and are never used.
        rc->x_bytes = (uint32_t)((x_bytes + 3) & ~3L);
        rc->off_bytes = (uint32_t)((off_bytes + 3) & ~3L);
        rc->mask_bytes = (uint32_t)((mask_bytes + 3) & ~3L);
        return true;
    };
    // For a target number of items per step, try group sets from all groups
    // down; take the first that fits with one workgroup per CU.
    auto try_plan = [&](int target) -> bool {
        const int max_thr = target > 448 ? 1024 : 512;
        for (int gs = G.g; gs >= 1; --gs) {
            if (G.g % gs) continue;
            const int items_row = G.wo * gs;
            if (items_row > max_thr) continue;
            int tr = (target + items_row - 1) / items_row;
            tr = std::max(1, std::min(tr, std::min(max_thr / items_row, G.ho)));
            if (fit(gs, tr, max_thr, num_cus, lds_limit, max_thr > 512 ? 16 : 8)) return true;
        }
        return false;
    };
    // Two workgroups per CU, each with half the LDS and at most 512 threads
    // of the 128-register kernel: while one loads its window the other
    // computes.
    auto try_pair = [&]() -> bool {
        for (int gs = G.g; gs >= 1; --gs) {
            if (G.g % gs) continue;
            const int items_row = G.wo * gs;
            if (items_row > 512) continue;
            const int tr = std::max(1, std::min((448 + items_row - 1) / items_row, std::min(512 / items_row, G.ho)));
            if (fit(gs, tr, 512, 2L * num_cus, lds_limit / 2, 16)) return true;
        }
        return false;
    };
    // A 1024-thread workgroup (four waves per SIMD, <= 128 VGPRs: a tap's
    // 32-byte corners and the item's offsets fit) hides the LDS latency
    // better than 512 threads; try that first.
    if (!(try_plan(896) || try_plan(448))) return false;
    // Where a workgroup of that plan walks a single step, its window load is
    // not overlapped with any compute; two workgroups per CU then overlap
    // one's loads with the other's step.
    if ((rc->chunk_rows + rc->tr - 1) / rc->tr <= 1) {
        const RingCfg one = *rc;
        if (try_pair() && rc->nwg >= 2L * num_cus) return true;
        *rc = one;
    }
    return true;
}

void device_limits(int* lds_limit, int* num_cus)
{
    static int cached_lds[64], cached_cus[64];
    static bool ready[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!__atomic_load_n(&ready[dev], __ATOMIC_ACQUIRE)) {
        // On a failed query keep conservative defaults: the planners then
        // size for 64 KB of LDS, which every gfx9 part provides.
        int lds = 65536, cus = 256;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 65536;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached_lds[dev] = lds;
        cached_cus[dev] = cus;
        __atomic_store_n(&ready[dev], true, __ATOMIC_RELEASE);
    }
    *lds_limit = cached_lds[dev];
    *num_cus = cached_cus[dev];
}

#ifdef DCN_COUNT_WRITES
DCN_WRITE_COUNT_SETTER(ring_count_writes)
#endif

}  // namespace dcn
