// DCN forward for f16, LDS sliding window of horizontally paired cells, for
// gfx950.
//
// Same operator as dcn_forward.hip ("DCNv4: Unbounded Weights", "Why Is
// Sampling Just 9 Points Still Slow?": y_g(p0) = sum_k m_gk x_g(p0 + p_k +
// dp_gk); bilinear reads with zero outside the map per "InternImage:
// Deformable Convolutions at Scale", Ch.2; softmax over K for DCNv3, Ch.3),
// and the same sliding-window scheme as dcn_forward_ring.hip: a workgroup
// owns one image, a set of channel groups and a chunk of output rows, keeps a
// ring of input rows in LDS and walks down its rows, a few per step.
//
// What differs is the cell stored in LDS.  The bilinear read of channel c at
// a tap is (1-b)[(1-a) X(y0,x0) + a X(y0,x0+1)] + b[(1-a) X(y0+1,x0) +
// a X(y0+1,x0+1)].  Each ring row holds, for every column x in [-1, W-1] and
// channel c, the 32-bit pair (X(x, c), X(x+1, c)) of 16-bit values (zero
// outside the map), so one tap of one channel is two v_dot2c_f32_f16 against
// the packed weight pairs ((1-a)(1-b)m, a(1-b)m) and ((1-a)bm, abm) instead
// of four multiply-adds: products and sums are fp32; the weights are rounded
// to f16 (relative error 2^-11) before the products.  (The same scheme in
// bf16 would round the weights to 2^-9 and spend most of the f16/bf16 error
// budget, so bf16 stays on the plain ring kernel.)
//
// A row is NQ planes of PS bytes (both compile-time): plane q holds the
// 16-byte chunk q (channels 4q..4q+3) of every (cell, group).  A wave's
// lanes, which read the same chunk of nearby cells in one instruction, then
// touch consecutive 16-byte slots, spread over all LDS bank groups; and the
// eight reads of a tap (NQ chunks of the top and of the bottom row) share
// one address with immediate offsets q*PS and NQ*PS + q*PS.
//
// The pairs cannot come straight from the buffer-to-LDS path, so each thread
// loads 16-byte runs of two neighbouring pixels into registers while a step
// computes, interleaves them with v_perm_b32 at the end of the step and
// writes the cells of the rows the next step adds.  Each lane also loads the
// offsets and modulation of its item of the next step straight into
// registers, so the whole LDS budget goes to the ring: at 16 channels per
// group that is what lets two groups share a workgroup on 56-pixel rows.
// Samples whose rows fall outside the window are read from global memory in
// a tail pass.
#include "dcn_device.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr uint32_t OOB = 0x80000000u;   // buffer offset past any accepted tensor: reads as zero
constexpr int CV_IT = 4;                // cell-conversion tasks per thread per step
constexpr int INIT_IT = 4;              // rounds of cell conversion for the first window

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

// Packed weight pairs and the two-term dot product, per storage type.
template <int DT> struct Pair;
template <> struct Pair<DT_F16> {
    static __device__ __forceinline__ uint32_t pack(float lo, float hi)
    {
        const f2_t v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2_t));
    }
    static __device__ __forceinline__ float dot(uint32_t x, uint32_t w, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, x), __builtin_bit_cast(h2_t, w), acc, false);
    }
};

template <int DT>
__device__ __forceinline__ float h2f(uint32_t h16)
{
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
    return __uint_as_float(h16 << 16);
}

// acc[0..8) += w * (16 bytes of x = 8 channels in the storage type)
template <int DT>
__device__ __forceinline__ void fma8(float* acc, float w, u32x4 r)
{
    const uint32_t q[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w, h2f<DT>(q[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, h2f<DT>(q[i] >> 16), acc[2 * i + 1]);
    }
}

// The 8 paired dwords of channels 8h..8h+7 of one cell from the 16-byte runs
// of those channels at pixel x (lo) and pixel x + 1 (hi).
__device__ __forceinline__ void interleave(u32x4 lo, u32x4 hi, u32x4& c0, u32x4& c1)
{
    c0.x = __builtin_amdgcn_perm(hi.x, lo.x, 0x05040100u);
    c0.y = __builtin_amdgcn_perm(hi.x, lo.x, 0x07060302u);
    c0.z = __builtin_amdgcn_perm(hi.y, lo.y, 0x05040100u);
    c0.w = __builtin_amdgcn_perm(hi.y, lo.y, 0x07060302u);
    c1.x = __builtin_amdgcn_perm(hi.z, lo.z, 0x05040100u);
    c1.y = __builtin_amdgcn_perm(hi.z, lo.z, 0x07060302u);
    c1.z = __builtin_amdgcn_perm(hi.w, lo.w, 0x05040100u);
    c1.w = __builtin_amdgcn_perm(hi.w, lo.w, 0x07060302u);
}

// NQ = 16-byte chunks of one paired cell row of a group (D / 4): 2 or 4;
// PS = bytes of one plane of a ring row.
template <int DT, bool SOFTMAX, int NQ, int PS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void dcn_fwd_pair(
    Geom G, RingCfg rc, const typename Elem<DT>::T* __restrict__ x, const typename Elem<DT>::T* __restrict__ off,
    const typename Elem<DT>::T* __restrict__ mask, typename Elem<DT>::T* __restrict__ out)
{
    using T = typename Elem<DT>::T;
    constexpr int ES = 2;
    constexpr int D = NQ * 4;                // channels per group
    constexpr int KH = 3, KW = 3, KF = 9;
    constexpr uint32_t K2B = KF * 2 * ES;    // offset bytes of one item
    constexpr uint32_t KMB = KF * ES;        // mask bytes of one item
    constexpr int HPC = D / 8;               // conversion tasks (8 channels each) per cell of one group
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
    const uint32_t gsize = (uint32_t)D * ES;            // global bytes of one group of a pixel
    constexpr uint32_t PITCH = NQ * PS;                 // bytes of one ring row

    // ---- cell conversion tasks: task t of a row is (cell, group, half of
    // the group's channels); this thread's tasks are t = tid + i * nthr over
    // the rows one step adds (the same tasks every step).
    const int tasks_row = (G.w + 1) * rc.gs * HPC;
    uint32_t cv_dst[CV_IT], cv_src[CV_IT];   // LDS offset within a slot; source offset within a row (or OOB)
    uint32_t cv_src2[CV_IT];                 // source of the right-hand pixel (or OOB)
    int cv_row[CV_IT];                       // row index among the step's new rows, or -1
#pragma unroll
    for (int i = 0; i < CV_IT; ++i) {
        const int t = tid + i * nthr;
        const int r = t / tasks_row, u = t - r * tasks_row;
        const int cellg = u / HPC, h = u - cellg * HPC;
        const int cell = cellg / rc.gs, gl = cellg - cell * rc.gs;
        const int xl = cell - 1;                         // left pixel of the pair
        cv_row[i] = i < rc.row_iters && r < adv ? r : -1;
        cv_dst[i] = (uint32_t)cell * rc.pb + 16u * gl + 2u * PS * h;
        const uint32_t so = (uint32_t)(g0 + gl) * gsize + 16u * h;
        cv_src[i] = xl >= 0 ? (uint32_t)xl * pix_g + so : OOB;
        cv_src2[i] = xl + 1 < G.w ? (uint32_t)(xl + 1) * pix_g + so : OOB;
    }
    u32x4 cv_lo[CV_IT], cv_hi[CV_IT];
    // Issue the loads of the cells of input row `row` for task i.
    auto cv_load = [&](int i, int row) {
        const bool inside = (unsigned)row < (unsigned)G.h;
        const uint32_t base = n * img_bytes + (uint32_t)row * row_bytes;
        cv_lo[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, inside && cv_src[i] != OOB ? base + cv_src[i] : OOB, 0, 0);
        cv_hi[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, inside && cv_src2[i] != OOB ? base + cv_src2[i] : OOB, 0, 0);
    };
    auto cv_store = [&](int i, int slot) {
        u32x4 c0, c1;
        interleave(cv_lo[i], cv_hi[i], c0, c1);
        unsigned char* d = ring + slot * PITCH + cv_dst[i];
        *reinterpret_cast<u32x4*>(d) = c0;
        *reinterpret_cast<u32x4*>(d + PS) = c1;
        if (slot == 0) {   // slot R mirrors slot 0
            unsigned char* m = ring + rc.R * PITCH + cv_dst[i];
            *reinterpret_cast<u32x4*>(m) = c0;
            *reinterpret_cast<u32x4*>(m + PS) = c1;
        }
    };

    // This lane's item within every step: row rl of the step, column c, group gl of the set.
    const int items_row = G.wo * rc.gs;
    const int rl = tid / items_row;
    const int rem = tid - rl * items_row;
    const int c = rem / rc.gs, gl = rem - c * rc.gs;
    const int g = g0 + gl;

    // Offsets and mask of this lane's item in a step, loaded into registers
    // one step ahead: the 9 dwords of its offset pairs and the 5 dwords that
    // hold its 9 modulation scalars (a run of 16-bit values that starts at
    // byte 0 or 2 of its first dword).
    uint32_t po[KF], pmr[5], psh = 0;
    auto load_offsets = [&](int s) {
        const int rr = r_begin + s * rc.tr + rl;
        const bool v = rl < rc.tr && rr < r_end;
        const uint32_t item = ((uint32_t)(n * G.ho + rr) * G.wo + c) * G.g + g;
        const uint32_t ob = v ? item * K2B : OOB;
        const uint32_t mb = v ? (item * KMB) & ~3u : OOB;
        psh = ((item * KMB) & 3u) * 8u;
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(orr, ob, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(orr, ob + 16u, 0, 0);
        po[0] = a.x; po[1] = a.y; po[2] = a.z; po[3] = a.w;
        po[4] = b.x; po[5] = b.y; po[6] = b.z; po[7] = b.w;
        po[8] = __builtin_amdgcn_raw_buffer_load_b32(orr, ob + 32u, 0, 0);
        const u32x4 mq = __builtin_amdgcn_raw_buffer_load_b128(mr, mb, 0, 0);
        pmr[0] = mq.x; pmr[1] = mq.y; pmr[2] = mq.z; pmr[3] = mq.w;
        pmr[4] = __builtin_amdgcn_raw_buffer_load_b32(mr, mb + 16u, 0, 0);
    };

    // ---- the first window: rows lo0 .. lo0 + nw - 1 in slots 0 .. nw - 1
    // (all of its loads in flight at once: INIT_IT rounds of adv rows cover it)
    load_offsets(0);
    {
        u32x4 in_lo[INIT_IT][CV_IT], in_hi[INIT_IT][CV_IT];
#pragma unroll
        for (int rr = 0; rr < INIT_IT; ++rr) {
#pragma unroll
            for (int i = 0; i < CV_IT; ++i) {
                const int wr = rr * adv + cv_row[i];
                if (cv_row[i] >= 0 && wr < rc.nw) {
                    cv_load(i, lo0 + wr);
                    in_lo[rr][i] = cv_lo[i];
                    in_hi[rr][i] = cv_hi[i];
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < INIT_IT; ++rr) {
#pragma unroll
            for (int i = 0; i < CV_IT; ++i) {
                const int wr = rr * adv + cv_row[i];
                if (cv_row[i] >= 0 && wr < rc.nw) {
                    cv_lo[i] = in_lo[rr][i];
                    cv_hi[i] = in_hi[rr][i];
                    cv_store(i, wr);
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const uint32_t gbyte = 16u * gl;
    const float lim = 16777216.0f;
    // Cell column (x0 + 1) and window row of each tap's top-left corner before the offset.
    int bxk[KW], byk[KH];
#pragma unroll
    for (int kx = 0; kx < KW; ++kx) bxk[kx] = c * G.sw - G.pw + 1 + kx * G.dw;
#pragma unroll
    for (int ky = 0; ky < KH; ++ky) byk[ky] = (r_begin + rl) * G.sh - G.ph - lo0 + ky * G.dh;

    int new_slot = rc.nw % rc.R;   // slot of the first row the next step adds
    for (int s = 0; s < nsteps; ++s) {
        const int r_s = r_begin + s * rc.tr;
        const int r = r_s + rl;
        const bool live = rl < rc.tr && r < r_end;
        const int lo = lo0 + s * adv;
        const int slot_lo = (s * adv) % rc.R;
        const bool more = s + 1 < nsteps;

        // ---- offsets and mask of this lane's item, then the next step's loads
        float dx[KF], dy[KF], m[KF];
        {
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                dx[k] = h2f<DT>(po[k] & 0xffffu);
                dy[k] = h2f<DT>(po[k] >> 16);
            }
            uint32_t mw[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) mw[i] = __builtin_amdgcn_alignbit(i < 4 ? pmr[i + 1] : 0u, pmr[i], psh);
#pragma unroll
            for (int k = 0; k < KF; ++k) m[k] = h2f<DT>((k & 1) ? mw[k >> 1] >> 16 : mw[k >> 1] & 0xffffu);
        }
        if (more) {
            load_offsets(s + 1);
#pragma unroll
            for (int i = 0; i < CV_IT; ++i)
                if (cv_row[i] >= 0) cv_load(i, lo + rc.nw + cv_row[i]);
        }

        float acc[D];
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
#pragma unroll
            for (int q = 0; q < D; ++q) acc[q] = 0.f;
            // Geometry of all taps: the LDS address of chunk 0 of the top
            // cell (chunk q is q planes further, the bottom cell one row
            // further) and the two packed weight pairs.
            uint32_t A[KF], WT[KF], WB[KF];
            uint32_t fb = 0;
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int kx = k / KH, ky = k - (k / KH) * KH;
                const float tx = fminf(fmaxf(G.scale * dx[k], -lim), lim);
                const float ty = fminf(fmaxf(G.scale * dy[k], -lim), lim);
                const float fx = floorf(tx), fy = floorf(ty);
                const float a = tx - fx, b = ty - fy;
                const int xs = bxk[kx] + (int)fx;                   // cell of the left corners, x0 + 1
                const int yi = byk[ky] + (int)fy;                   // window row of the top corners
                const bool colok = (unsigned)xs <= (unsigned)G.w;   // image column x0 in [-1, W-1]
                const bool inwin = (unsigned)yi < (unsigned)(rc.nw - 1);
                fb |= (colok && !inwin) ? (1u << k) : 0u;
                const bool use = colok && inwin;
                uint32_t s0 = (uint32_t)(slot_lo + yi);
                s0 = min(s0, s0 - (uint32_t)rc.R);                  // wrap once
                const uint32_t addr = s0 * PITCH + __umul24((uint32_t)xs, (uint32_t)rc.pb) + gbyte;
                A[k] = use ? addr : 0u;
                const float mm = use ? m[k] : 0.f;
                const float ma = mm * (1.f - a), mb = mm * a;
                WT[k] = Pair<DT>::pack(ma * (1.f - b), mb * (1.f - b));
                WB[k] = Pair<DT>::pack(ma * b, mb * b);
            }
            // Reads of tap k+1 are in flight while tap k accumulates.
            u32x4 cur[2 * NQ], nxt[2 * NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                cur[q] = *reinterpret_cast<const u32x4*>(ring + A[0] + PS * q);
                cur[NQ + q] = *reinterpret_cast<const u32x4*>(ring + A[0] + PITCH + PS * q);
            }
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                if (k + 1 < KF) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        nxt[q] = *reinterpret_cast<const u32x4*>(ring + A[k + 1] + PS * q);
                        nxt[NQ + q] = *reinterpret_cast<const u32x4*>(ring + A[k + 1] + PITCH + PS * q);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the next tap's reads ahead of this tap's math
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const uint32_t t4[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
                    const uint32_t b4[4] = {cur[NQ + q].x, cur[NQ + q].y, cur[NQ + q].z, cur[NQ + q].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[4 * q + j] = Pair<DT>::dot(t4[j], WT[k], acc[4 * q + j]);
                        acc[4 * q + j] = Pair<DT>::dot(b4[j], WB[k], acc[4 * q + j]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (k + 1 < KF) {
#pragma unroll
                    for (int q = 0; q < 2 * NQ; ++q) cur[q] = nxt[q];
                }
            }
            // Tail: samples outside the window that may touch the image, read
            // from global memory, each lane walking only its own such taps;
            // the tap's offsets and modulation are read again from global
            // memory (the staging area has been released).
            if (fb) {
                const uint32_t base_img = n * img_bytes + (uint32_t)g * gsize;
                const uint32_t item = ((uint32_t)(n * G.ho + r) * G.wo + c) * G.g + g;
                while (fb) {
                    const int k = __builtin_ctz(fb);
                    fb &= fb - 1u;
                    const int kx = k / KH, ky = k - kx * KH;
                    const uint32_t pr = __builtin_amdgcn_raw_buffer_load_b32(orr, item * K2B + 4u * k, 0, 0);
                    const float dxk = h2f<DT>(pr & 0xffffu), dyk = h2f<DT>(pr >> 16);
                    float mk = h2f<DT>(__builtin_amdgcn_raw_buffer_load_b16(mr, item * KMB + 2u * k, 0, 0));
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
                    const uint32_t o00 = (cy0 && cx0) ? p00 : OOB, o01 = (cy0 && cx1) ? p00 + pix_g : OOB;
                    const uint32_t o10 = (cy1 && cx0) ? p00 + row_bytes : OOB;
                    const uint32_t o11 = (cy1 && cx1) ? p00 + row_bytes + pix_g : OOB;
                    const float ma = mk * (1.f - a), mb = mk * a;
#pragma unroll
                    for (int h = 0; h < D / 8; ++h) {
                        fma8<DT>(acc + 8 * h, ma * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o00 + 16u * h, 0, 0));
                        fma8<DT>(acc + 8 * h, mb * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o01 + 16u * h, 0, 0));
                        fma8<DT>(acc + 8 * h, ma * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o10 + 16u * h, 0, 0));
                        fma8<DT>(acc + 8 * h, mb * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o11 + 16u * h, 0, 0));
                    }
                }
            }
        }

        // ---- cells of the rows the next step adds (their slots are not read by this step)
        if (more) {
#pragma unroll
            for (int i = 0; i < CV_IT; ++i) {
                if (cv_row[i] >= 0) {
                    int slot = new_slot + cv_row[i];
                    if (slot >= rc.R) slot -= rc.R;
                    cv_store(i, slot);
                }
            }
            new_slot += adv;
            if (new_slot >= rc.R) new_slot -= rc.R;
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's buffer-to-LDS loads and cell writes have landed
        // The outputs are stored after that wait, so that it never waits for
        // this step's stores; the next step's wait covers them.
        if (live) {
            T* op = out + (((long)(n * G.ho + r) * G.wo + c) * G.c + (long)g * D);
#pragma unroll
            for (int h = 0; h < D / 8; ++h) store_vec<DT>(op + 8 * h, acc + 8 * h);
        }
        __syncthreads();
    }
}

template <int DT, bool SOFTMAX>
hipError_t launch_pair_typed(const Geom& G, const RingCfg& rc, const void* x, const void* off, const void* mask,
                             void* out, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const dim3 grid(rc.nwg), block(rc.threads);
#define DCN_PAIR_CASE(NQV, PSV)                                                                               \
    case NQV * 8192 + PSV: {                                                                                  \
        auto* fn = dcn_fwd_pair<DT, SOFTMAX, NQV, PSV>;                                                       \
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,        \
                                           rc.lds_bytes);                                                     \
        if (e != hipSuccess) return e;                                                                        \
        fn<<<grid, block, rc.lds_bytes, s>>>(G, rc, (const T*)x, (const T*)off, (const T*)mask, (T*)out);      \
        break;                                                                                                \
    }
    switch (G.d / 4 * 8192 + rc.pitch / (G.d / 4)) {
        DCN_PAIR_CASE(2, 1024)
        DCN_PAIR_CASE(2, 2048)
        DCN_PAIR_CASE(4, 1024)
        DCN_PAIR_CASE(4, 2048)
        default: return hipErrorInvalidValue;
    }
#undef DCN_PAIR_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_forward_pair(const Geom& G, const RingCfg& rc, int dtype, const void* x, const void* off,
                                   const void* mask, void* out, hipStream_t s)
{
    switch (dtype * 2 + (G.softmax ? 1 : 0)) {
        case DT_F16 * 2 + 0: return launch_pair_typed<DT_F16, false>(G, rc, x, off, mask, out, s);
        case DT_F16 * 2 + 1: return launch_pair_typed<DT_F16, true>(G, rc, x, off, mask, out, s);
    }
    return hipErrorInvalidValue;
}

// Choose the group set, rows per step, halo and chunking of the paired-cell
// kernel for geometry G, or return false when it does not apply (f16, 3x3,
// D of 8 or 16, 16-byte aligned tensors).
bool plan_pair(const Geom& G, int dtype, const void* x, const void* off, const void* mask, const void* out,
               int lds_limit, int num_cus, RingCfg* rc)
{
    if (dtype != DT_F16) return false;
    if (G.kh != 3 || G.kw != 3) return false;
    if (G.d != 8 && G.d != 16) return false;
    if ((uintptr_t)x % 16 || (uintptr_t)off % 16 || (uintptr_t)mask % 16 || (uintptr_t)out % 16) return false;
    const int es = 2;
    const long x_bytes = (long)G.n * G.h * G.w * G.c * es;
    const long off_bytes = (long)G.items * G.K * 2 * es, mask_bytes = (long)G.items * G.K * es;
    if (x_bytes >= (1L << 31) || off_bytes >= (1L << 31) - 64 || mask_bytes >= (1L << 31) - 64) return false;
    const int HPC = G.d / 8;

    const int HY_MIN = 3, HY_MAX = 8;
    for (int gs = G.g; gs >= 1; --gs) {
        if (G.g % gs) continue;
        const int items_row = G.wo * gs;
        if (items_row > 512) continue;
        int tr = (448 + items_row - 1) / items_row;
        tr = std::max(1, std::min(tr, std::min(512 / items_row, G.ho)));
        const int items_step = tr * items_row;
        const int threads = std::max(64, (items_step + 63) / 64 * 64);
        const int pb = gs * 16;                         // bytes of one cell in one plane (gs groups)
        const int nq = G.d / 4;
        const long plane_need = (long)(G.w + 1) * pb;
        if (plane_need > 2048) continue;
        const int ps = plane_need <= 1024 ? 1024 : 2048;   // plane size, a kernel template parameter
        const long pitch = (long)nq * ps;
        const int adv = tr * G.sh;
        const long tasks_row = (long)(G.w + 1) * gs * HPC;
        const int cv_iters = (int)((adv * tasks_row + threads - 1) / threads);
        if (cv_iters > 4) continue;   // CV_IT
        int hy = -1, nw = 0, R = 0;
        for (int h = HY_MAX; h >= HY_MIN; --h) {
            const int nwh = (tr - 1) * G.sh + (G.kh - 1) * G.dh + 2 + 2 * h;
            const int Rh = nwh + adv;
            if (nwh > 4 * adv) continue;   // INIT_IT rounds fill the first window
            if ((long)(Rh + 1) * pitch <= lds_limit) {
                hy = h;
                nw = nwh;
                R = Rh;
                break;
            }
        }
        if (hy < 0) continue;
        const int gsets = G.g / gs;
        const long units = (long)G.n * gsets;
        int chunks = (int)std::max(1L, ((long)num_cus + units - 1) / units);
        chunks = std::min(chunks, (G.ho + tr - 1) / tr);
        int chunk_rows = (G.ho + chunks - 1) / chunks;
        chunk_rows = (chunk_rows + tr - 1) / tr * tr;
        chunks = (G.ho + chunk_rows - 1) / chunk_rows;
        if (units * chunks >= (1L << 31)) continue;
        rc->gs = gs;
        rc->gsets = gsets;
        rc->pb = pb;
        rc->cpp = 0;
        rc->pitch = (int)pitch;
        rc->R = R;
        rc->nw = nw;
        rc->hy = hy;
        rc->tr = tr;
        rc->chunk_rows = chunk_rows;
        rc->chunks = chunks;
        rc->nwg = (int)(units * chunks);
        rc->threads = threads;
        rc->row_iters = cv_iters;   // conversion tasks per thread per step
        rc->st_contig = 0;   // no staging area: offsets and mask go to registers
        rc->cpo = 0;
        rc->cpm = 0;
        rc->stage_o_bytes = 0;
        rc->ring_bytes = (int)((R + 1) * pitch);
        rc->lds_bytes = rc->ring_bytes;
        // Buffer loads range-check each dword; see plan_ring.
        rc->x_bytes = (uint32_t)((x_bytes + 3) & ~3L);
        rc->off_bytes = (uint32_t)((off_bytes + 3) & ~3L);
        rc->mask_bytes = (uint32_t)((mask_bytes + 3) & ~3L);
        return true;
    }
    return false;
}

}  // namespace dcn
