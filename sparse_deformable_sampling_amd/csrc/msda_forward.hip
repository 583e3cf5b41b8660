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
// Locations come either as given normalised (u, v) per sample, or are formed
// here from a reference per query and an offset per sample ("Deformable
// DETR...", "A reference links resolutions without equating their pixels" and
// "Math and tensor shapes"), in fp64:
//  - point reference (x, y):  u = x r_w + dx / W_l,  v = y r_h + dy / H_l;
//  - box reference (x, y, w, h):  u = x r_w + (dx / P) w r_w / 2, likewise v;
// with (r_w, r_h) the level's valid ratios of the image (1 when absent).  An
// optional padding mask marks value cells as padded; they read zero, as the
// attention module zeroes projected values at masked positions.
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

// Where the sample locations come from.  REF = 0: `loc` holds (u, v) per
// sample.  REF = 2 or 4: `loc` holds the per-sample offsets (same layout),
// `ref` the per-query point or box, `ratio` [n][L][2] valid ratios (or NULL).
// `pad` [n][S] marks padded value cells (or NULL).
struct MsdaSrc {
    const float* loc;
    const float* ref;
    const float* ratio;
    const uint8_t* pad;
};

// Normalised location (u, v) of sample i (level l) of item (n, q, head), fp64.
// `rat`, when given, holds image n's valid ratios per level (else they are
// read from src.ratio).
template <int REF>
__device__ __forceinline__ void sample_uv(const MsdaGeom& G, const MsdaSrc& src, int n, int q, long item, int l, int i,
                                          double& u, double& v, const float2* rat = nullptr)
{
    const int LP = G.L * G.P;
    const float2 t = *reinterpret_cast<const float2*>(src.loc + (item * LP + i) * 2);
    if constexpr (REF == 0) {
        u = t.x;
        v = t.y;
    } else {
        const float* r = src.ref + ((long)n * G.q + q) * REF;
        double rw = 1.0, rh = 1.0;
        if (rat) {
            rw = rat[l].x;
            rh = rat[l].y;
        } else if (src.ratio) {
            rw = src.ratio[((long)n * G.L + l) * 2];
            rh = src.ratio[((long)n * G.L + l) * 2 + 1];
        }
        // Reciprocals instead of fp64 divisions: one extra rounding of 2^-53.
        if constexpr (REF == 2) {
            u = (double)r[0] * rw + (double)t.x * G.inv_w[l];
            v = (double)r[1] * rh + (double)t.y * G.inv_h[l];
        } else {
            u = (double)r[0] * rw + (double)t.x * G.half_inv_p * (double)r[2] * rw;
            v = (double)r[1] * rh + (double)t.y * G.half_inv_p * (double)r[3] * rh;
        }
    }
}

// Whether value cell `cell` (index within the image's S cells) of image n is padded.
__device__ __forceinline__ bool padded(const MsdaSrc& src, const MsdaGeom& G, int n, long cell)
{
    return src.pad && src.pad[(long)n * G.S + cell] != 0;
}

__device__ __forceinline__ Sample sample_geometry(const MsdaGeom& G, const MsdaSrc& src, int n, int l, double u,
                                                  double v, float A, long img_head)
{
    Sample s;
    s.any = false;
    const int Hl = G.H[l], Wl = G.W[l];
    const double x = u * Wl - 0.5, y = v * Hl - 0.5;
    if (!(x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl)) return s;
    const double fx = floor(x), fy = floor(y);
    const float a = (float)(x - fx), b = (float)(y - fy);
    const int x0 = (int)fx, y0 = (int)fy;
    const long cell = (long)G.start[l] + (long)y0 * Wl + x0;
    s.c00 = y0 >= 0 && x0 >= 0 && !padded(src, G, n, cell);
    s.c01 = y0 >= 0 && x0 + 1 < Wl && !padded(src, G, n, cell + 1);
    s.c10 = y0 + 1 < Hl && x0 >= 0 && !padded(src, G, n, cell + Wl);
    s.c11 = y0 + 1 < Hl && x0 + 1 < Wl && !padded(src, G, n, cell + Wl + 1);
    const float Aa = A * (1.f - a), Ab = A * a;
    s.w00 = Aa * (1.f - b);
    s.w01 = Ab * (1.f - b);
    s.w10 = Aa * b;
    s.w11 = Ab * b;
    s.base = img_head + ((long)G.start[l] + (long)y0 * Wl + x0) * G.m * G.dh;
    s.any = true;
    return s;
}

// Padding of value cells `byte` and `byte + 1` (byte offsets into the [n][S]
// mask): bit 0 for the first, bit 1 for the second (a nonzero byte is padded).
// One 8-byte load from the dword that holds the first byte covers both; a
// dword past the mask reads zero, and neither cell is then used.
__device__ __forceinline__ uint32_t pad_pair(__amdgpu_buffer_rsrc_t pr, uint32_t byte)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(pr, byte & ~3u, 0, 0);
    const uint32_t two = __builtin_amdgcn_alignbit(w.y, w.x, (byte & 3u) * 8u);   // the two bytes, low first
    return ((two & 0xffu) != 0u ? 1u : 0u) | ((two & 0xff00u) != 0u ? 2u : 0u);
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
template <bool SOFTMAX, int REF>
__global__ __launch_bounds__(256) void msda_fwd_vec4(MsdaGeom G, const float* __restrict__ value, MsdaSrc src,
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
    const int q = (int)((item / G.m) % G.q);
    const int LP = G.L * G.P;
    const float* ai = attn + item * LP;
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
            double u, vv;
            sample_uv<REF>(G, src, n, q, item, l, i, u, vv);
            const Sample s = sample_geometry(G, src, n, l, u, vv, A, img_head);
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
// Sample records per workgroup: up to 512 (16 KB of LDS), so that 8
// workgroups share a CU; with two samples' corners in flight per lane (48
// VGPRs) that is 8 waves per SIMD.  1024 records and four samples in flight
// ran at 5 waves per SIMD and took 428 us against 369 us at the encoder shape.
// A workgroup has at least one query's samples per thread row (the softmax
// shuffles span them), which takes up to 1024 records at 32 samples per head.
constexpr int MS_REC_MAX = 512;

// Queries per workgroup of the tiled kernel for LP samples and LQ lanes per query.
inline int tile_queries(int LP, int LQ)
{
    int QT = std::min(256 / LQ, MS_REC_MAX / LP);
    if (QT * LQ < LP) QT = LP / LQ;
    return QT;
}

template <bool SOFTMAX, int REF>
__global__ __launch_bounds__(256) void msda_fwd_tile(MsdaGeom G, int LPlog, int LQlog, int QT, int tiles, int nwg,
                                                     uint32_t value_bytes, const float* __restrict__ value,
                                                     MsdaSrc src, const float* __restrict__ attn,
                                                     float* __restrict__ out)
{
    // LDS: QT*LP corner offsets, QT*LP weights, and (references only) per level
    // the image's valid ratio times the level's extent, (r_w W_l, r_h H_l)
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4* rec_o = reinterpret_cast<u32x4*>(lds);
    float4* rec_w = reinterpret_cast<float4*>(lds + (size_t)(QT << LPlog) * 16);
    double* rsc = reinterpret_cast<double*>(lds + (size_t)(QT << LPlog) * 32);
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

    if constexpr (REF != 0) {
        if (tid < 2 * G.L) {
            const int l = tid >> 1, ax = tid & 1;   // ax 0: width, 1: height
            const double r = src.ratio ? (double)src.ratio[((long)n * G.L + l) * 2 + ax] : 1.0;
            rsc[tid] = r * (double)(ax ? G.H[l] : G.W[l]);   // exact: a 24-bit by <= 24-bit product
        }
        __syncthreads();
    }

    // ---- phase 1: sample records
    // The padding mask (references only) through a buffer resource: two cell
    // pairs per sample, (y0, x0..x0+1) and (y0+1, x0..x0+1), one 8-byte load each.
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)src.pad, (short)0, (int)((((long)G.n * G.S) + 3) & ~3L), 0x00020000);
    const int nsamp = QT << LPlog;
    for (int s = tid; s < nsamp; s += nthr) {
        const int qi = s >> LPlog, i = s & (LP - 1);
        const int q = q0 + qi;
        const bool valid = q < G.q;
        const int qc = valid ? q : 0;
        const long item = ((long)n * G.q + qc) * G.m + h;
        float A = attn[item * LP + i];
        if constexpr (SOFTMAX) {
            float mx = A;
            mx = group_reduce<true>(mx, LP);
            const float e = exp_nonpos(A - mx);
            float sum = e;
            sum = group_reduce<false>(sum, LP);
            A = e * (1.0f / sum);
        }
        const int l = i / G.P;
        const int Hl = G.H[l], Wl = G.W[l];
        u32x4 o = {MS_OOB, MS_OOB, MS_OOB, MS_OOB};
        float4 w = {0.f, 0.f, 0.f, 0.f};
        // Pixel coordinates x = u W_l - 1/2, y = v H_l - 1/2, in fp64.  With a
        // reference, u W_l is written out: x = x_ref (r_w W_l) + dx for a point,
        // x = (r_w W_l)(x_ref + dx w / (2P)) for a box (the offset term of u
        // times W_l), each one or two fp64 FMAs of exact products.
        double x, y;
        {
            const float2 t = *reinterpret_cast<const float2*>(src.loc + (item * LP + i) * 2);
            if constexpr (REF == 0) {
                x = (double)t.x * Wl - 0.5;
                y = (double)t.y * Hl - 0.5;
            } else {
                const float* r = src.ref + ((long)n * G.q + qc) * REF;
                const double sw = rsc[2 * l], sh = rsc[2 * l + 1];
                if constexpr (REF == 2) {
                    x = fma((double)r[0], sw, (double)t.x - 0.5);
                    y = fma((double)r[1], sh, (double)t.y - 0.5);
                } else {
                    x = fma(sw, fma((double)t.x * (double)r[2], G.half_inv_p, (double)r[0]), -0.5);
                    y = fma(sh, fma((double)t.y * (double)r[3], G.half_inv_p, (double)r[1]), -0.5);
                }
            }
        }
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
            uint32_t padm = 0;   // bits: 00, 01, 10, 11 corners padded
            if (REF != 0 && src.pad) {
                const uint32_t byte = (uint32_t)((long)n * G.S + G.start[l] + (long)y0 * Wl + x0);
                padm = pad_pair(pr, byte) | (pad_pair(pr, byte + (uint32_t)Wl) << 2);
            }
            o.x = (cy0 && cx0 && !(padm & 1u)) ? base : MS_OOB;
            o.y = (cy0 && cx1 && !(padm & 2u)) ? base + unit : MS_OOB;
            o.z = (cy1 && cx0 && !(padm & 4u)) ? base + down : MS_OOB;
            o.w = (cy1 && cx1 && !(padm & 8u)) ? base + down + unit : MS_OOB;
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
#pragma unroll 2
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
template <bool SOFTMAX, int REF>
__global__ __launch_bounds__(256) void msda_fwd_generic(MsdaGeom G, const float* __restrict__ value, MsdaSrc src,
                                                        const float* __restrict__ attn, float* __restrict__ out)
{
    const long item = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long items = (long)G.n * G.q * G.m;
    if (item >= items) return;
    const int h = (int)(item % G.m);
    const int n = (int)(item / ((long)G.q * G.m));
    const int q = (int)((item / G.m) % G.q);
    const int LP = G.L * G.P;
    const float* ai = attn + item * LP;
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
            double u, v;
            sample_uv<REF>(G, src, n, q, item, l, i, u, v);
            const Sample s = sample_geometry(G, src, n, l, u, v, A, img_head);
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

namespace {

template <int REF>
hipError_t launch_src(const MsdaGeom& G, const float* value, const MsdaSrc& src, const float* attn, float* out,
                      hipStream_t s)
{
    const long items = (long)G.n * G.q * G.m;
    const bool aligned = ((uintptr_t)value % 16 == 0) && ((uintptr_t)out % 16 == 0) && ((uintptr_t)src.loc % 8 == 0);
    const dim3 block(256);
    const int LP = G.L * G.P, LQ = G.dh / 4;
    const long value_bytes = (long)G.n * G.S * G.m * G.dh * 4;
    const bool pow2 = (LP & (LP - 1)) == 0 && LP <= 32 && G.dh % 4 == 0 && (LQ & (LQ - 1)) == 0 && LQ <= 64;
    if (aligned && pow2 && value_bytes < (1L << 31) - 64) {
        int LPlog = 0, LQlog = 0;
        while ((1 << LPlog) < LP) ++LPlog;
        while ((1 << LQlog) < LQ) ++LQlog;
        const int QT = tile_queries(LP, LQ);
        const int tiles = (G.q + QT - 1) / QT;
        const long nwg = (long)G.n * G.m * tiles;
        if (nwg < (1L << 30)) {
            const dim3 grid((unsigned)((nwg + 7) & ~7L)), blk((unsigned)(QT * LQ));
            const size_t lds = (size_t)QT * LP * 32 + MSDA_MAX_LEVELS * 2 * sizeof(double);
            if (G.softmax)
                msda_fwd_tile<true, REF><<<grid, blk, lds, s>>>(G, LPlog, LQlog, QT, tiles, (int)nwg,
                                                                (uint32_t)value_bytes, value, src, attn, out);
            else
                msda_fwd_tile<false, REF><<<grid, blk, lds, s>>>(G, LPlog, LQlog, QT, tiles, (int)nwg,
                                                                 (uint32_t)value_bytes, value, src, attn, out);
            return hipGetLastError();
        }
    }
    if (aligned && G.dh % 4 == 0) {
        const long lanes = items * (G.dh / 4);
        const dim3 grid((unsigned)((lanes + 255) / 256));
        if (G.softmax) msda_fwd_vec4<true, REF><<<grid, block, 0, s>>>(G, value, src, attn, out);
        else msda_fwd_vec4<false, REF><<<grid, block, 0, s>>>(G, value, src, attn, out);
    } else {
        const dim3 grid((unsigned)((items + 255) / 256));
        if (G.softmax) msda_fwd_generic<true, REF><<<grid, block, 0, s>>>(G, value, src, attn, out);
        else msda_fwd_generic<false, REF><<<grid, block, 0, s>>>(G, value, src, attn, out);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_msda_forward(const MsdaGeom& G, const float* value, const float* loc, const float* attn, float* out,
                               hipStream_t s)
{
    const MsdaSrc src = {loc, nullptr, nullptr, nullptr};
    return launch_src<0>(G, value, src, attn, out, s);
}

hipError_t launch_msda_forward_ref(const MsdaGeom& G, int ref_dims, const float* value, const float* ref,
                                   const float* ratios, const float* offsets, const float* attn,
                                   const uint8_t* pad, float* out, hipStream_t s)
{
    const MsdaSrc src = {offsets, ref, ratios, pad};
    return ref_dims == 4 ? launch_src<4>(G, value, src, attn, out, s) : launch_src<2>(G, value, src, attn, out, s);
}

#ifdef DCN_COUNT_WRITES
DCN_WRITE_COUNT_SETTER(msda_count_writes)
#endif

}  // namespace dcn
