// DCN forward, LDS sliding-window kernel for gfx950.
//
// Same operator as dcn_forward.hip ("DCNv4: Unbounded Weights", "Why Is
// Sampling Just 9 Points Still Slow?": y_g(p0) = sum_k m_gk x_g(p0 + p_k +
// dp_gk), bilinear reads with zero outside the map per "InternImage:
// Deformable Convolutions at Scale", Ch.2; softmax over K for DCNv3, Ch.3).
//
// Why a different kernel: on gfx950 a scattered 16-32 byte read through the
// vector L1 costs about one cache-line lookup (~2.3 clocks per line per CU),
// so gathering 36 corners per output from L1 runs far below HBM speed.  The
// LDS serves the same random 16-byte reads 6x faster.  Each workgroup
// therefore owns one image and a chunk of output rows, keeps a ring of input
// rows (all channels, one zero column on each side) in LDS, and walks down
// the chunk TR output rows per step:
//   - the window of input rows a step can touch without leaving the ring is
//     [lo, lo + NW): the rows the 3x3 footprint reaches plus HY halo rows
//     above and below for the learned offsets;
//   - while a step computes, the rows the next step adds and the next step's
//     offsets and mask are already in flight to registers, then written to
//     LDS before the step's closing barrier;
//   - a sample whose two rows fall outside the window but touch the image is
//     rare (|dy| > HY); it is skipped in the LDS pass and read with global
//     loads in a tail pass by the lanes that need it.
// Lane = one (output pixel, group) item holding all D channels, so the tap
// geometry is computed once per item and reused for every channel; fp32
// accumulation; stores are 16-byte vectors, one writer per element.
#include "dcn_device.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr uint32_t OOB = 0x80000000u;   // buffer offset past any accepted tensor: reads as zero

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ u32x4 lds_ld16(const unsigned char* base, uint32_t off)
{
    return *reinterpret_cast<const u32x4*>(base + off);
}

template <int DT>
__device__ __forceinline__ void fma16(float* acc, float w, u32x4 r)
{
    const uint32_t q[4] = {r.x, r.y, r.z, r.w};
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

template <int DT>
__device__ __forceinline__ float half_lo(uint32_t p)
{
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu));
    return __uint_as_float(p << 16);
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t p)
{
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
    return __uint_as_float(p & 0xffff0000u);
}

// One wave copies `bytes` (a multiple of 16) from a buffer into LDS at
// `dst`, 1 KB per instruction: lane l of the wave lands at dst + c + 16*l.
// `src` == OOB copies zeros.  The wave's share is every nwaves-th kilobyte.
__device__ __forceinline__ void wave_copy_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t src, unsigned char* dst,
                                                 uint32_t bytes, int wave, int nwaves, int lane)
{
    for (uint32_t c = (uint32_t)wave * 1024u; c < bytes; c += (uint32_t)nwaves * 1024u) {
        const uint32_t o = c + 16u * lane;
        if (o < bytes)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + c), 16, src == OOB ? OOB : src + o, 0, 0, 0);
    }
}

template <int DT, int KH, int KW, bool SOFTMAX, int NCH>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void dcn_fwd_ring(Geom G, RingCfg rc, const typename Elem<DT>::T* __restrict__ x,
                                                    const typename Elem<DT>::T* __restrict__ off,
                                                    const typename Elem<DT>::T* __restrict__ mask,
                                                    typename Elem<DT>::T* __restrict__ out)
{
    using T = typename Elem<DT>::T;
    constexpr int ES = sizeof(T);
    constexpr int V = 16 / ES;               // channels per 16-byte chunk
    constexpr int KF = KH * KW;
    static_assert(KF > 0, "ring kernel is instantiated for fixed kernels");
    static_assert(ES == 2, "ring kernel stages 16-bit offsets and mask");
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* ring = lds;
    unsigned char* stage = lds + rc.ring_bytes;

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    int L = blockIdx.x;
    if (rc.nwg % 8 == 0) L = (blockIdx.x % 8) * (rc.nwg / 8) + blockIdx.x / 8;   // neighbours share an XCD
    const int n = L / rc.chunks, chunk = L - n * rc.chunks;
    const int r_begin = chunk * rc.chunk_rows;
    const int r_end = min(G.ho, r_begin + rc.chunk_rows);
    if (r_begin >= r_end) return;
    const int nsteps = (r_end - r_begin + rc.tr - 1) / rc.tr;
    const int adv = rc.tr * G.sh;                       // window advance per step (input rows)
    const int lo0 = r_begin * G.sh - G.ph - rc.hy;      // first row of the first window

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)rc.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc((void*)off, (short)0, (int)rc.off_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc((void*)mask, (short)0, (int)rc.mask_bytes, 0x00020000);
    const uint32_t img_bytes = (uint32_t)G.h * G.w * G.c * ES;
    const uint32_t row_bytes = (uint32_t)G.w * G.c * ES;

    // Input row `row` into its ring slot (zeros outside the image).
    // Slot R mirrors slot 0, so the row below any slot is always the next slot in memory.
    auto load_row = [&](int row) {
        const int slot = (row - lo0) % rc.R;
        const uint32_t src = (unsigned)row < (unsigned)G.h ? n * img_bytes + (uint32_t)row * row_bytes : OOB;
        wave_copy_to_lds(xr, src, ring + slot * rc.pitch + rc.pb, row_bytes, wave, nwaves, lane);
        if (slot == 0) wave_copy_to_lds(xr, src, ring + rc.R * rc.pitch + rc.pb, row_bytes, wave, nwaves, lane);
    };
    // Offsets and mask of one step's items: the items of a step are
    // contiguous, so both runs are staged with aligned 16-byte loads.
    auto stage_range = [&](int s, uint32_t& o_lo, uint32_t& m_lo, uint32_t& o_len, uint32_t& m_len) {
        const int r_s = r_begin + s * rc.tr;
        const int rows = min(rc.tr, r_end - r_s);
        const uint32_t first = ((uint32_t)(n * G.ho + r_s) * G.wo) * G.g;
        const uint32_t cnt = (uint32_t)rows * G.wo * G.g;
        const uint32_t ob = first * KF * 2 * ES, oe = (first + cnt) * KF * 2 * ES;
        const uint32_t mb = first * KF * ES, me = (first + cnt) * KF * ES;
        o_lo = ob & ~15u;
        m_lo = mb & ~15u;
        o_len = ((oe + 15u) & ~15u) - o_lo;
        m_len = ((me + 15u) & ~15u) - m_lo;
    };
    auto load_stage = [&](int s) {
        uint32_t o_lo, m_lo, o_len, m_len;
        stage_range(s, o_lo, m_lo, o_len, m_len);
        wave_copy_to_lds(orr, o_lo, stage, o_len, wave, nwaves, lane);
        wave_copy_to_lds(mr, m_lo, stage + o_len, m_len, wave, nwaves, lane);
    };

    // Zero the two border columns of every ring slot (never written again).
    {
        const int pbc = rc.pb / 16;
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < (rc.R + 1) * 2 * pbc; i += nthr) {
            const int slot = i / (2 * pbc), j = i - slot * 2 * pbc;
            const uint32_t col_off = j < pbc ? 16u * j : (uint32_t)(G.w + 1) * rc.pb + 16u * (j - pbc);
            *reinterpret_cast<u32x4*>(ring + slot * rc.pitch + col_off) = z;
        }
    }
    for (int rr = 0; rr < rc.nw; ++rr) load_row(lo0 + rr);
    load_stage(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int items_row = G.wo * G.g;
    const float lim = 16777216.0f;

    for (int s = 0; s < nsteps; ++s) {
        const int r_s = r_begin + s * rc.tr;
        const int rows_s = min(rc.tr, r_end - r_s);
        const int lo = lo0 + s * adv;
        const int slot_lo = (s * adv) % rc.R;

        // ---- this lane's item; its offsets and mask come out of the staging area
        const int i = tid;
        const bool live = i < rows_s * items_row;
        const int rl = live ? i / items_row : 0;
        const int rem = live ? i - rl * items_row : 0;
        const int c = rem / G.g, g = rem - c * G.g;
        const int r = r_s + rl;
        uint32_t dxy[KF];
        float m[KF];
        {
            uint32_t o_lo, m_lo, o_len, m_len;
            stage_range(s, o_lo, m_lo, o_len, m_len);
            const uint32_t item = ((uint32_t)(n * G.ho + r) * G.wo + c) * G.g + g;
            const uint32_t ob = item * KF * 2 * ES - o_lo;
            const uint32_t mb = o_len + item * KF * ES - m_lo;
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                dxy[k] = *reinterpret_cast<const uint32_t*>(stage + ob + 4u * k);
                const uint16_t h = *reinterpret_cast<const uint16_t*>(stage + mb + 2u * k);
                m[k] = half_lo<DT>((uint32_t)h);
            }
        }
        __syncthreads();   // the staging area is free for the next step

        // ---- the next step's new rows and staging data go straight to LDS
        if (s + 1 < nsteps) {
            for (int rr = 0; rr < adv; ++rr) load_row(lo + rc.nw + rr);
            load_stage(s + 1);
        }

        // ---- compute this lane's item from the ring
        if (live) {
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
            }
            float acc[NCH * V];
#pragma unroll
            for (int q = 0; q < NCH * V; ++q) acc[q] = 0.f;
            // Geometry of all taps first: one LDS address (top-left corner, the
            // other three are +pb, +pitch, +pitch+pb) and four weights per tap.
            const int bx = c * G.sw - G.pw, by = r * G.sh - G.ph;
            const int bx1 = bx + 1;                        // LDS column of tap column 0 (image column + 1)
            const int byw = r * G.sh - G.ph - lo;          // window row of tap row 0
            const uint32_t gbyte = (uint32_t)g * G.d * ES;
            uint32_t A[KF];
            float W00[KF], W01[KF], W10[KF], W11[KF];
            uint32_t fb = 0;
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int kx = k / KH, ky = k - (k / KH) * KH;
                const float tx = fminf(fmaxf(G.scale * half_lo<DT>(dxy[k]), -lim), lim);
                const float ty = fminf(fmaxf(G.scale * half_hi<DT>(dxy[k]), -lim), lim);
                const float fx = floorf(tx), fy = floorf(ty);
                const float a = tx - fx, b = ty - fy;
                int xs = bx1 + kx * G.dw + (int)fx;                 // column of the left corners, +1
                int yi = byw + ky * G.dh + (int)fy;                 // window row of the top corners
                const bool colok = (unsigned)xs <= (unsigned)G.w;   // image column in [-1, W-1]
                const bool inwin = (unsigned)yi < (unsigned)(rc.nw - 1);
                fb |= (colok && !inwin) ? (1u << k) : 0u;
                const bool use = colok && inwin;
                const float mm = use ? m[k] : 0.f;
                xs = use ? xs : 0;
                yi = use ? yi : 0;
                uint32_t s0 = (uint32_t)(slot_lo + yi);
                s0 = min(s0, s0 - (uint32_t)rc.R);                  // wrap once
                A[k] = __umul24(s0, (uint32_t)rc.pitch) + __umul24((uint32_t)xs, (uint32_t)rc.pb) + gbyte;
                const float ma = mm * (1.f - a), mb = mm * a;
                W00[k] = ma * (1.f - b);
                W01[k] = mb * (1.f - b);
                W10[k] = ma * b;
                W11[k] = mb * b;
            }
            // Reads of tap k+1 are in flight while tap k accumulates.
            const uint32_t o01 = (uint32_t)rc.pb, o10 = (uint32_t)rc.pitch, o11 = (uint32_t)(rc.pitch + rc.pb);
            u32x4 cur[4 * NCH], nxt[4 * NCH];
#pragma unroll
            for (int q = 0; q < NCH; ++q) {
                cur[4 * q + 0] = lds_ld16(ring, A[0] + 16u * q);
                cur[4 * q + 1] = lds_ld16(ring, A[0] + o01 + 16u * q);
                cur[4 * q + 2] = lds_ld16(ring, A[0] + o10 + 16u * q);
                cur[4 * q + 3] = lds_ld16(ring, A[0] + o11 + 16u * q);
            }
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                if (k + 1 < KF) {
#pragma unroll
                    for (int q = 0; q < NCH; ++q) {
                        nxt[4 * q + 0] = lds_ld16(ring, A[k + 1] + 16u * q);
                        nxt[4 * q + 1] = lds_ld16(ring, A[k + 1] + o01 + 16u * q);
                        nxt[4 * q + 2] = lds_ld16(ring, A[k + 1] + o10 + 16u * q);
                        nxt[4 * q + 3] = lds_ld16(ring, A[k + 1] + o11 + 16u * q);
                    }
                }
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
            // Tail: samples outside the window but touching the image, read from global memory.
            if (fb) {
                const uint32_t base_img = n * img_bytes + gbyte;
                const uint32_t pixb = (uint32_t)G.c * ES;
                for (int k = 0; k < KF; ++k) {
                    if (!((fb >> k) & 1u)) continue;
                    const int kx = k / KH, ky = k - (k / KH) * KH;
                    const float tx = fminf(fmaxf(G.scale * half_lo<DT>(dxy[k]), -lim), lim);
                    const float ty = fminf(fmaxf(G.scale * half_hi<DT>(dxy[k]), -lim), lim);
                    const float fx = floorf(tx), fy = floorf(ty);
                    const float a = tx - fx, b = ty - fy;
                    const int x0 = bx + kx * G.dw + (int)fx;
                    const int y0 = by + ky * G.dh + (int)fy;
                    const bool cx0 = (unsigned)x0 < (unsigned)G.w, cx1 = (unsigned)(x0 + 1) < (unsigned)G.w;
                    const bool cy0 = (unsigned)y0 < (unsigned)G.h, cy1 = (unsigned)(y0 + 1) < (unsigned)G.h;
                    const uint32_t p00 = base_img + ((uint32_t)y0 * G.w + (uint32_t)x0) * pixb;
                    const uint32_t o00 = (cy0 && cx0) ? p00 : OOB, o01 = (cy0 && cx1) ? p00 + pixb : OOB;
                    const uint32_t o10 = (cy1 && cx0) ? p00 + row_bytes : OOB;
                    const uint32_t o11 = (cy1 && cx1) ? p00 + row_bytes + pixb : OOB;
                    const float ma = m[k] * (1.f - a), mb = m[k] * a;
#pragma unroll
                    for (int q = 0; q < NCH; ++q) {
                        fma16<DT>(acc + q * V, ma * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o00 + 16u * q, 0, 0));
                        fma16<DT>(acc + q * V, mb * (1.f - b), __builtin_amdgcn_raw_buffer_load_b128(xr, o01 + 16u * q, 0, 0));
                        fma16<DT>(acc + q * V, ma * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o10 + 16u * q, 0, 0));
                        fma16<DT>(acc + q * V, mb * b, __builtin_amdgcn_raw_buffer_load_b128(xr, o11 + 16u * q, 0, 0));
                    }
                }
            }
            T* op = out + (((long)(n * G.ho + r) * G.wo + c) * G.c + (long)g * G.d);
#pragma unroll
            for (int q = 0; q < NCH; ++q) store_vec<DT>(op + q * V, acc + q * V);
        }

        __builtin_amdgcn_s_waitcnt(0);   // this wave's direct-to-LDS loads have landed
        __syncthreads();
    }
}

template <int DT, bool SOFTMAX>
hipError_t launch_ring_typed(const Geom& G, const RingCfg& rc, const void* x, const void* off, const void* mask,
                             void* out, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const int nch = G.d * (int)sizeof(T) / 16;
    const dim3 grid(rc.nwg), block(rc.threads);
#define DCN_RING_CASE(NCHV)                                                                                   \
    case NCHV: {                                                                                              \
        auto* fn = dcn_fwd_ring<DT, 3, 3, SOFTMAX, NCHV>;                                                     \
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,        \
                                           rc.lds_bytes);                                                     \
        if (e != hipSuccess) return e;                                                                        \
        fn<<<grid, block, rc.lds_bytes, s>>>(G, rc, (const T*)x, (const T*)off, (const T*)mask, (T*)out);      \
        break;                                                                                                \
    }
    switch (nch) {
        DCN_RING_CASE(1)
        DCN_RING_CASE(2)
        DCN_RING_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef DCN_RING_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_forward_ring(const Geom& G, const RingCfg& rc, int dtype, const void* x, const void* off,
                                   const void* mask, void* out, hipStream_t s)
{
    switch (dtype * 2 + (G.softmax ? 1 : 0)) {
        case DT_F16 * 2 + 0: return launch_ring_typed<DT_F16, false>(G, rc, x, off, mask, out, s);
        case DT_F16 * 2 + 1: return launch_ring_typed<DT_F16, true>(G, rc, x, off, mask, out, s);
        case DT_BF16 * 2 + 0: return launch_ring_typed<DT_BF16, false>(G, rc, x, off, mask, out, s);
        case DT_BF16 * 2 + 1: return launch_ring_typed<DT_BF16, true>(G, rc, x, off, mask, out, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn

namespace dcn {

bool plan_ring(const Geom& G, int dtype, const void* x, const void* off, const void* mask, const void* out,
               int lds_limit, int num_cus, RingCfg* rc)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    if (G.kh != 3 || G.kw != 3) return false;
    const int es = 2;
    const int nch = G.d * es / 16;
    if (G.d * es % 16 != 0 || (nch != 1 && nch != 2 && nch != 4)) return false;
    if ((uintptr_t)x % 16 || (uintptr_t)off % 16 || (uintptr_t)mask % 16 || (uintptr_t)out % 16) return false;
    const long x_bytes = (long)G.n * G.h * G.w * G.c * es;
    const long off_bytes = (long)G.items * G.K * 2 * es, mask_bytes = (long)G.items * G.K * es;
    if (x_bytes >= (1L << 31) || off_bytes >= (1L << 31) - 64 || mask_bytes >= (1L << 31) - 64) return false;
    const int items_row = G.wo * G.g;
    if (items_row > 512) return false;
    int tr = (384 + items_row - 1) / items_row;
    tr = std::max(1, std::min(tr, std::min(512 / items_row, G.ho)));
    const int items_step = tr * items_row;
    const int threads = (items_step + 63) / 64 * 64;
    const int pb = G.c * es;
    const long pitch = (long)(G.w + 2) * pb + 16;
    const int stage_bytes = 16 * ((items_step * G.K * 2 * es + 15) / 16 + 2 + (items_step * G.K * es + 15) / 16 + 2);
    const int adv = tr * G.sh;
    int hy = -1, nw = 0, R = 0;
    for (int h = 8; h >= 2; --h) {
        const int nwh = (tr - 1) * G.sh + (G.kh - 1) * G.dh + 2 + 2 * h;
        const int Rh = nwh + adv;
        if ((long)(Rh + 1) * pitch + stage_bytes <= lds_limit) {
            hy = h;
            nw = nwh;
            R = Rh;
            break;
        }
    }
    if (hy < 0) return false;
    int chunks = std::max(1, (num_cus + G.n - 1) / G.n);
    chunks = std::min(chunks, (G.ho + tr - 1) / tr);
    int chunk_rows = (G.ho + chunks - 1) / chunks;
    chunk_rows = (chunk_rows + tr - 1) / tr * tr;
    chunks = (G.ho + chunk_rows - 1) / chunk_rows;
    if ((long)G.n * chunks >= (1L << 31)) return false;
    rc->pb = pb;
    rc->pitch = (int)pitch;
    rc->R = R;
    rc->nw = nw;
    rc->hy = hy;
    rc->tr = tr;
    rc->chunk_rows = chunk_rows;
    rc->chunks = chunks;
    rc->nwg = G.n * chunks;
    rc->threads = threads;
    rc->ring_bytes = (int)((R + 1) * pitch);
    rc->lds_bytes = rc->ring_bytes + stage_bytes;
    // Buffer loads range-check each dword: a dword that straddles num_records
    // reads as zero.  Rounding the extents up to whole dwords keeps the last
    // values of an odd-length f16 tensor readable; the extra bytes share a
    // dword (and so a page) with valid data and are never used.
    rc->x_bytes = (uint32_t)((x_bytes + 3) & ~3L);
    rc->off_bytes = (uint32_t)((off_bytes + 3) & ~3L);
    rc->mask_bytes = (uint32_t)((mask_bytes + 3) & ~3L);
    return true;
}

void device_limits(int* lds_limit, int* num_cus)
{
    static int cached_lds[64], cached_cus[64];
    static bool ready[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!__atomic_load_n(&ready[dev], __ATOMIC_ACQUIRE)) {
        int lds = 65536, cus = 256;
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        cached_lds[dev] = lds;
        cached_cus[dev] = cus;
        __atomic_store_n(&ready[dev], true, __ATOMIC_RELEASE);
    }
    *lds_limit = cached_lds[dev];
    *num_cus = cached_cus[dev];
}

}  // namespace dcn
