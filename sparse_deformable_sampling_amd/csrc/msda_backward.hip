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
//  - Phase 2, lane = (query, 4 channels) (1 channel below head_dim 4): for
//    every sample, read the four corners' 16-byte slices, scatter A*w*g into
//    grad_value with buffer atomics (a query's lanes add to one contiguous
//    run, the access pattern fp32 atomics serve fastest; out-of-range corners
//    are dropped by the buffer range check), and reduce the three channel
//    sums across the query's lanes with DPP moves; the query's first lane
//    writes (dL/du, dL/dv, A, dL/dA) back into the sample's LDS record.
//  - Phase 3, one thread per sample: softmax backward over the query's
//    samples, coalesced stores of grad_loc and grad_attn.
//
// With a workspace, grad_value is a gather instead of a scatter.  The value
// gradient of a cell is a sum over the samples whose four corners include it,
// so the samples are first grouped by cell (a counting sort per (image, head)
// pair) and each cell then reads its own samples and writes its gradient
// once: no atomics and no zero-fill.
//  - Bucket of a sample: the cell (x0, y0) = (floor x, floor y) of its corner
//    with the smallest coordinates, on a grid of (H_l+1) x (W_l+1) per level
//    (x0, y0 >= -1 for a sample inside the level's extended range).  Cell
//    (x, y) is a corner of the samples of buckets x0 in {x-1, x}, y0 in
//    {y-1, y}: two runs of two adjacent buckets, contiguous in bucket order.
//  - msda_bwd_count_lds: a workgroup counts 8192 samples of one pair per
//    bucket in LDS (the returned count is the rank among them), then adds
//    each nonzero count to the pair's global count with one atomic, whose
//    return is the workgroup's base; a sample's rank is base + local rank.
//    msda_bwd_count, one global atomic per sample, serves pairs whose
//    buckets do not fit in LDS.
//  - msda_bwd_scan: exclusive prefix sum of the counts, one workgroup per
//    pair, through LDS where the pair's counts fit.
//  - the tiled kernel writes each sample's record (query, A, a, b) at
//    offset + rank, alongside grad_loc and grad_attn.
//  - msda_bwd_cells: a group of head_dim/4 lanes per block of 4 adjacent
//    cells of a row, 4 channels a lane; the group reads the block's two runs
//    of records in batches (one record per lane, the 4 cells' weights formed
//    by the lane that read it, broadcast through LDS) and the matching
//    16-byte slices of grad_out, and stores the 4 sums.  Coarse levels, whose
//    cells have the longest runs, are dispatched first.
#include <algorithm>

#include "dcn_device.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr uint32_t MS_OOB = 0x80000000u;
// Sample records per workgroup of the tiled kernel: up to 512 (16 KB of LDS),
// more only where one query's samples need it (see tile_queries).
constexpr int MS_REC_MAX = 512;

// Buckets of the value-gradient gather (see above).
struct MsdaSortCfg {
    int Sp;                                // buckets per pair: sum of (H_l+1)(W_l+1); offsets hold Sp+1
    int pstart[MSDA_MAX_LEVELS];           // first bucket of level l within a pair
    int wg_per_pair[MSDA_MAX_LEVELS];      // cell-kernel workgroups per pair at level l
    int gpc[MSDA_MAX_LEVELS];              // lane groups per block of cells at level l (a power of two)
    int blk_start[MSDA_MAX_LEVELS + 1];    // first cell-kernel workgroup of the k-th level taken (coarsest
                                           // first), each a multiple of 8; the last is the grid size
};

// Pixel coordinate of a sample on a level of W x H cells (cell centres at
// integers, formed in fp64), its top-left corner (x0, y0) and fractions.
// False when no corner lies inside the level.
__device__ __forceinline__ bool msda_corner(float2 uv, int Wl, int Hl, int& x0, int& y0, float& fa, float& fb)
{
    const double x = (double)uv.x * Wl - 0.5, y = (double)uv.y * Hl - 0.5;
    if (!(x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl)) return false;
    const double fx = floor(x), fy = floor(y);
    fa = (float)(x - fx);
    fb = (float)(y - fy);
    x0 = (int)fx;
    y0 = (int)fy;
    return true;
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float lane_sum(float v, int width)
{
    for (int o = 1; o < width; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over aligned groups of `w` lanes (a power of two up to 64): DPP moves
// within a row of 16 (swap neighbours, then pairs, then mirror within 8 and
// within 16 lanes), cross-lane shuffles beyond; every lane of a group ends
// with the group's sum.
__device__ __forceinline__ float row_sum(float v, int w)
{
    if (w >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
    if (w >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
    if (w >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half-row mirror
    if (w >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)); // row mirror
    if (w >= 32) v += __shfl_xor(v, 16, 64);
    if (w >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// V consecutive fp32 values at byte offset o (zeros past the buffer's end).
template <int V>
__device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t r, uint32_t o, float* v)
{
    if constexpr (V == 4) {
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    } else {
        v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0));
    }
}

// SORTED: write each sample's record for the gather (records, offsets and
// ranks as described above) instead of adding into grad_value.
// V channels per lane in phase 2: 4 for the gather (head_dim >= 4), else 1,
// so that each atomic instruction covers a query's whole run of channels.
template <bool SOFTMAX, bool SORTED, int V>
__global__ __launch_bounds__(256) void msda_bwd_tile(MsdaGeom G, int LPlog, int Dlog, int QT, int tiles, int nwg,
                                                     uint32_t value_bytes, const float* __restrict__ value,
                                                     const float* __restrict__ loc, const float* __restrict__ attn,
                                                     const float* __restrict__ gout, float* __restrict__ gvalue,
                                                     float* __restrict__ gloc, float* __restrict__ gattn,
                                                     MsdaSortCfg C, const int* __restrict__ boff,
                                                     const int* __restrict__ rank, int4* __restrict__ rec)
{
    // LDS: QT*LP corner offsets, then QT*LP (a, b, A) / gradient records
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4* rec_o = reinterpret_cast<u32x4*>(lds);
    float4* rec_f = reinterpret_cast<float4*>(lds + (size_t)(QT << LPlog) * 16);
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
            mx = group_reduce<true>(mx, LP);
            const float e = exp_nonpos(A - mx);
            float sum = e;
            sum = group_reduce<false>(sum, LP);
            A = e * (1.0f / sum);
        }
        const int l = i / G.P;
        const int Hl = G.H[l], Wl = G.W[l];
        u32x4 o = {MS_OOB, MS_OOB, MS_OOB, MS_OOB};
        float fa = 0.f, fb = 0.f;
        int x0, y0;
        if (msda_corner(uv, Wl, Hl, x0, y0, fa, fb) && valid) {
            if constexpr (SORTED) {
                const int bk = C.pstart[l] + (y0 + 1) * (Wl + 1) + x0 + 1;
                const int pos = boff[(long)pair * (C.Sp + 1) + bk] + rank[item * LP + i];
                rec[((long)pair * G.q << LPlog) + pos] = make_int4(q, __float_as_int(A), __float_as_int(fa),
                                                                   __float_as_int(fb));
            }
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

    // ---- phase 2: lane = (query, V channels)
    {
        const int LPQ = G.dh / V;   // lanes per query
        const int qi = tid / LPQ, c = tid - qi * LPQ;
        const int q = q0 + qi;
        const bool live = qi < QT && q < G.q;
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)value, (short)0, (int)value_bytes,
                                                                            0x00020000);
        const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc((void*)gvalue, (short)0,
                                                                            gvalue ? (int)value_bytes : 0, 0x00020000);
        const long item = ((long)n * G.q + (live ? q : 0)) * G.m + h;
        float g[V];
#pragma unroll
        for (int k = 0; k < V; ++k) g[k] = live ? gout[item * G.dh + V * c + k] : 0.f;
        const uint32_t cb = 4u * V * c;
        const int r0 = (live ? qi : 0) << LPlog;
        // Lanes of a query that is past the end still take part in the
        // reductions (with g = 0) and write nothing.  The corners of U
        // samples are loaded before any is used (U = 2 for the gather, whose
        // loop is otherwise latency-bound; the scatter is bound by its atomics).
        constexpr int U = V == 4 ? 2 : 1;
        for (int i0 = 0; i0 < LP; i0 += U) {
            float vv[U][4][V];
            float4 ff[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = i0 + u < LP;
                const u32x4 o = in ? rec_o[r0 + i0 + u] : u32x4{MS_OOB, MS_OOB, MS_OOB, MS_OOB};
                ff[u] = in ? rec_f[r0 + i0 + u] : make_float4(0.f, 0.f, 0.f, 0.f);
                load_v<V>(vr, o.x + cb, vv[u][0]);
                load_v<V>(vr, o.y + cb, vv[u][1]);
                load_v<V>(vr, o.z + cb, vv[u][2]);
                load_v<V>(vr, o.w + cb, vv[u][3]);
                if constexpr (U == 1) {
                    if (gvalue && live) {
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            const float Ag = ff[u].z * g[k];
                            const float a = ff[u].x, bb = ff[u].y;
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * ((1.f - a) * (1.f - bb)), gr,
                                                                            o.x + cb + 4 * k, 0, 0);
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * (a * (1.f - bb)), gr,
                                                                            o.y + cb + 4 * k, 0, 0);
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * ((1.f - a) * bb), gr,
                                                                            o.z + cb + 4 * k, 0, 0);
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(Ag * (a * bb), gr, o.w + cb + 4 * k,
                                                                            0, 0);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u;
                const float a = ff[u].x, bb = ff[u].y, A = ff[u].z;
                const float* v00 = vv[u][0];
                const float* v01 = vv[u][1];
                const float* v10 = vv[u][2];
                const float* v11 = vv[u][3];
                const float wa = 1.f - a, wb = 1.f - bb;
                const float w00 = wa * wb, w01 = a * wb, w10 = wa * bb, w11 = a * bb;
                float sA = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    sA += g[k] * (w00 * v00[k] + w01 * v01[k] + w10 * v10[k] + w11 * v11[k]);
                    sa += g[k] * (wb * (v01[k] - v00[k]) + bb * (v11[k] - v10[k]));
                    sb += g[k] * (wa * (v10[k] - v00[k]) + a * (v11[k] - v01[k]));
                }
                const float dA = row_sum(sA, LPQ), da = row_sum(sa, LPQ), db = row_sum(sb, LPQ);
                if (live && c == 0 && i < LP) {
                    const int l = i / G.P;
                    rec_f[r0 + i] = make_float4(A * da * (float)G.W[l], A * db * (float)G.H[l], A, dA);
                }
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

// One thread per sample: count the sample into its bucket; the count before
// it is its rank (-1 for a sample with no corner inside its level).
__global__ __launch_bounds__(256) void msda_bwd_count(MsdaGeom G, MsdaSortCfg C, int LPlog,
                                                      const float* __restrict__ loc, int* __restrict__ cnt,
                                                      int* __restrict__ rank)
{
    const int s = blockIdx.x * 256 + threadIdx.x;
    if (s >= (G.n * G.q * G.m << LPlog)) return;
    const int item = s >> LPlog, i = s & ((1 << LPlog) - 1);
    const int h = item % G.m, n = item / (G.q * G.m);
    const int l = i / G.P;
    const float2 uv = *reinterpret_cast<const float2*>(loc + (long)s * 2);
    int x0, y0, r = -1;
    float fa, fb;
    if (msda_corner(uv, G.W[l], G.H[l], x0, y0, fa, fb)) {
        const int bk = C.pstart[l] + (y0 + 1) * (G.W[l] + 1) + x0 + 1;
        r = atomicAdd(cnt + (long)(n * G.m + h) * (C.Sp + 1) + bk, 1);
    }
    rank[s] = r;
}

// The same counts and ranks, aggregated in LDS first: a workgroup of 1024
// threads takes CQ_SAMPLES samples of one pair (CQ_SAMPLES / LP consecutive
// queries), counts them per bucket with LDS atomics (the returned value is
// the rank among the workgroup's samples), adds each nonzero bucket count to
// the global one with a single atomic (which returns the workgroup's base),
// and writes base + local rank.  Queries that are neighbours in the map
// share coarse-level buckets, so this replaces most global atomics on
// crowded addresses by LDS ones.  LDS: Sp ints (Sp < 2^15).
constexpr int CQ_SPT = 8;                   // samples per thread
constexpr int CQ_SAMPLES = 1024 * CQ_SPT;   // samples per workgroup
static_assert(CQ_SAMPLES <= (1 << 15), "local ranks are packed into 15 bits");

__global__ __launch_bounds__(1024) void msda_bwd_count_lds(MsdaGeom G, MsdaSortCfg C, int LPlog, int chunks,
                                                           const float* __restrict__ loc, int* __restrict__ cnt,
                                                           int* __restrict__ rank)
{
    extern __shared__ int lc[];
    const int pair = blockIdx.x / chunks, ck = blockIdx.x - pair * chunks;
    const int n = pair / G.m, h = pair - n * G.m;
    const int t = threadIdx.x;
    for (int b = t; b < C.Sp; b += 1024) lc[b] = 0;
    __syncthreads();
    const int LP = 1 << LPlog;
    // bucket * 2^15 + local rank, or -1: Sp < 2^15 (LDS) and ranks < CQ_SAMPLES <= 2^15
    int br[CQ_SPT];
#pragma unroll
    for (int k = 0; k < CQ_SPT; ++k) {
        const int sl = ck * CQ_SAMPLES + k * 1024 + t;
        const int q = sl >> LPlog, i = sl & (LP - 1);
        br[k] = -1;
        if (q < G.q) {
            const int l = i / G.P;
            const long gs = (((long)n * G.q + q) * G.m + h) * LP + i;
            const float2 uv = *reinterpret_cast<const float2*>(loc + gs * 2);
            int x0, y0;
            float fa, fb;
            if (msda_corner(uv, G.W[l], G.H[l], x0, y0, fa, fb)) {
                const int bk = C.pstart[l] + (y0 + 1) * (G.W[l] + 1) + x0 + 1;
                br[k] = (bk << 15) | atomicAdd(lc + bk, 1);
            }
        }
    }
    __syncthreads();
    int* gc = cnt + (long)pair * (C.Sp + 1);
    for (int b = t; b < C.Sp; b += 1024) {
        const int c = lc[b];
        if (c) lc[b] = atomicAdd(gc + b, c);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CQ_SPT; ++k) {
        const int sl = ck * CQ_SAMPLES + k * 1024 + t;
        const int q = sl >> LPlog, i = sl & (LP - 1);
        if (q < G.q) rank[(((long)n * G.q + q) * G.m + h) * LP + i] = br[k] >= 0 ? lc[br[k] >> 15] + (br[k] & 0x7fff) : -1;
    }
}

// In-place exclusive prefix sum of `len` counts per pair, one workgroup of
// 1024 threads per pair, each thread over a contiguous run.  STAGED: the
// pair's counts pass through LDS (len ints), so that global memory is read
// and written with coalesced accesses.
template <bool STAGED>
__global__ __launch_bounds__(1024) void msda_bwd_scan(int* __restrict__ cnt, int len)
{
    __shared__ int wsum[16];
    extern __shared__ int stg[];
    int* g = cnt + (long)blockIdx.x * len;
    int* p = g;
    if constexpr (STAGED) {
        for (int i = threadIdx.x; i < len; i += 1024) stg[i] = g[i];
        __syncthreads();
        p = stg;
    }
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int per = (len + 1023) / 1024;
    const int lo = min(len, t * per), hi = min(len, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += p[i];
    int v = sum;
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[wv] = v;
    __syncthreads();
    if (t < 64) {
        int w = t < 16 ? wsum[t] : 0;
        for (int o = 1; o < 16; o <<= 1) {
            const int u = __shfl_up(w, o, 64);
            if (lane >= o) w += u;
        }
        if (t < 16) wsum[t] = w;
    }
    __syncthreads();
    int run = (wv ? wsum[wv - 1] : 0) + v - sum;
    for (int i = lo; i < hi; ++i) {
        const int c = p[i];
        p[i] = run;
        run += c;
    }
    if constexpr (STAGED) {
        __syncthreads();
        for (int i = threadIdx.x; i < len; i += 1024) g[i] = stg[i];
    }
}

// grad_value by cells.  A group of LPC = head_dim/4 lanes (4 channels a
// lane) owns a block of CB adjacent cells of one row, x = xs .. xs+CB-1.
// Their samples lie in the buckets px = xs .. xs+CB (px = x0 + 1) of two
// bucket rows (py = y: the cells are the samples' lower corners, weight b;
// py = y+1: upper corners, 1-b), i.e. two contiguous runs of records.  A
// sample of bucket px adds (1-a) of itself to cell px-1 and a to cell px, so
// each record is read once for the whole block (CB+1 bucket columns instead
// of 2*CB for single cells).  Per batch every lane reads one record, finds
// its bucket from the run boundaries and forms the weights of the CB cells;
// the records' grad_out slices are then read and summed, the next batch's
// records already in flight.  A level whose blocks expect long runs gives
// each block gpc groups (interleaved batches), summed through LDS.
// A coarse cell gathers thousands of terms (about 1300 per head on the
// 13x17 level of the encoder shape), too many for one fp32 running sum to
// stay within 1e-5 of the exact sum.  So each round's LPC terms are summed
// in fp32 (a chain of LPC, about 2^-24 of relative error per term) and the
// round sums are added in fp64, which keeps the long chain's error at about
// 2^-53 per round.  (fp64 products for every term cost the kernel 35% more
// time; the short fp32 chains cost nothing measurable.)
constexpr int CB = 4;

template <int LPC>
__global__ __launch_bounds__(256) void msda_bwd_cells(MsdaGeom G, MsdaSortCfg C, int LPlog,
                                                      const int* __restrict__ boff, const int4* __restrict__ rec,
                                                      const float* __restrict__ gout, uint32_t gout_bytes,
                                                      float* __restrict__ gvalue)
{
    __shared__ float stage[CB + 1][256];   // per lane: grad_out offset, then the CB weights
    __shared__ double part[4][256];        // one cell's partial sums per lane, reduced cell by cell
    const int b = blockIdx.x;
    int k = 0;
    while (k + 1 < G.L && b >= C.blk_start[k + 1]) ++k;
    const int l = G.L - 1 - k;
    const int local = b - C.blk_start[k];
    const int nb = C.blk_start[k + 1] - C.blk_start[k];
    const int r = (local & 7) * (nb >> 3) + (local >> 3);   // each XCD sweeps a contiguous range
    const int wpp = C.wg_per_pair[l];
    const int pair = r / wpp;
    if (pair >= G.n * G.m) return;
    const int n = pair / G.m, h = pair - n * G.m;
    const int gpc = C.gpc[l];
    const int t = threadIdx.x, grp = t / LPC, j = t - grp * LPC;
    const int slot = grp / gpc, gi = grp - slot * gpc;
    const int Wl = G.W[l];
    const int nbx = (Wl + CB - 1) / CB;
    const int blk = (r - pair * wpp) * (256 / (LPC * gpc)) + slot;
    const bool live = blk < nbx * G.H[l];
    const int y = live ? blk / nbx : 0, xs = live ? (blk - y * nbx) * CB : 0;
    // run boundaries: bnd[row][i] = first record of bucket px = xs + i (i = 0 .. CB+1,
    // clamped to the row's end W+1, which is where the next row starts)
    const int* po = boff + (long)pair * (C.Sp + 1) + C.pstart[l] + y * (Wl + 1);
    int bu[CB + 2], bl[CB + 2];
#pragma unroll
    for (int i = 0; i < CB + 2; ++i) {
        const int px = min(xs + i, Wl + 1);
        bu[i] = po[px];
        bl[i] = po[Wl + 1 + px];
    }
    const int n0 = live ? bu[CB + 1] - bu[0] : 0;
    const int ntot = live ? n0 + bl[CB + 1] - bl[0] : 0;
    const int4* pr = rec + ((long)pair * G.q << LPlog);
    const uint32_t rowb = (uint32_t)G.m * G.dh * 4u;
    const uint32_t gbase = (uint32_t)((long)n * G.q * G.m + h) * (uint32_t)(G.dh * 4) + 16u * j;
    const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc((void*)gout, (short)0, (int)gout_bytes,
                                                                        0x00020000);
    const int step = gpc * LPC;
    auto index = [&](int tt) { return tt < n0 ? bu[0] + tt : bl[0] + tt - n0; };
    int4 e = make_int4(0, 0, 0, 0);
    if (gi * LPC + j < ntot) e = pr[index(gi * LPC + j)];
    double acc[CB][4];
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] = 0.0;
    for (int k0 = gi * LPC; k0 < ntot; k0 += step) {   // the same trip count for the whole group
        const int tt = k0 + j;
        float w[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) w[c] = 0.f;
        uint32_t go = MS_OOB;   // past the end of grad_out: reads zero
        if (tt < ntot) {
            const bool upper = tt < n0;
            const int idx = index(tt);
            int kb = 0;   // bucket of the record: px = xs + kb
#pragma unroll
            for (int i = 1; i <= CB; ++i) kb += idx >= (upper ? bu[i] : bl[i]);
            const float fa = __int_as_float(e.z), fb = __int_as_float(e.w);
            const float Aw = __int_as_float(e.y) * (upper ? fb : 1.f - fb);
            const float wl = Aw * (1.f - fa), wr = Aw * fa;   // to cells px-1 and px
#pragma unroll
            for (int c = 0; c < CB; ++c) w[c] = c == kb - 1 ? wl : (c == kb ? wr : 0.f);
            go = (uint32_t)e.x * rowb;
        }
        if (tt + step < ntot) e = pr[index(tt + step)];
        stage[0][t] = __uint_as_float(go);
#pragma unroll
        for (int c = 0; c < CB; ++c) stage[c + 1][t] = w[c];
        wave_lds_sync();
        // the LPC records of this round summed in fp32, the round's sum
        // added to the fp64 total (short fp32 chains, one fp64 add per
        // output and round instead of one fp64 product per record)
        float part32[CB][4];
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) part32[c][i] = 0.f;
#pragma unroll
        for (int u = 0; u < LPC; ++u) {
            const int src = grp * LPC + u;
            const uint32_t o = __float_as_uint(stage[0][src]);
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(gr, o == MS_OOB ? o : o + gbase, 0, 0);
            const float gv[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                 __uint_as_float(v.w)};
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const float ww = stage[c + 1][src];
#pragma unroll
                for (int i = 0; i < 4; ++i) part32[c][i] = fmaf(ww, gv[i], part32[c][i]);
            }
        }
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] += (double)part32[c][i];
        wave_lds_sync();
    }
    if (gpc > 1) {   // uniform over the workgroup
#pragma unroll
        for (int c = 0; c < CB; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i][t] = acc[c][i];
            __syncthreads();
            if (gi == 0)
                for (int u = 1; u < gpc; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[c][i] += part[i][t + u * LPC];
            __syncthreads();
        }
    }
    if (live && gi == 0) {
        float* dst = gvalue + (((long)n * G.S + G.start[l] + (long)y * Wl + xs) * G.m + h) * G.dh + 4 * j;
#pragma unroll
        for (int c = 0; c < CB; ++c)
            if (xs + c < Wl)
                *reinterpret_cast<float4*>(dst + (long)c * G.m * G.dh) =
                    make_float4((float)acc[c][0], (float)acc[c][1], (float)acc[c][2], (float)acc[c][3]);
    }
}

// Queries per workgroup of the tiled kernel: at most 256 lanes of V channels
// and MS_REC_MAX sample records, but at least one query's samples per thread
// row (the softmax shuffles of phases 1 and 3 span them): up to 1024 records
// at 32 samples per head.
int tile_queries(const MsdaGeom& G, int V)
{
    const int LP = G.L * G.P, LPQ = G.dh / V;
    int QT = std::min(256 / LPQ, MS_REC_MAX / LP);
    if (QT * LPQ < LP) QT = LP / LPQ;
    return QT;
}

// Shapes the tiled kernel takes (LPlog, Dlog filled in).
bool tile_shape(const MsdaGeom& G, const float* loc, const float* gloc, int* LPlog, int* Dlog)
{
    const int LP = G.L * G.P;
    const long value_bytes = (long)G.n * G.S * G.m * G.dh * 4;
    const bool aligned = (uintptr_t)loc % 8 == 0 && (!gloc || (uintptr_t)gloc % 8 == 0);
    const bool pow2 = (LP & (LP - 1)) == 0 && LP <= 32 && (G.dh & (G.dh - 1)) == 0 && G.dh <= 64;
    if (!aligned || !pow2 || value_bytes >= (1L << 31) - 64) return false;
    const int QT = tile_queries(G, 1);   // the smaller of the two tilings
    if ((long)G.n * G.m * ((G.q + QT - 1) / QT) >= (1L << 30)) return false;
    *LPlog = 0;
    *Dlog = 0;
    while ((1 << *LPlog) < LP) ++*LPlog;
    while ((1 << *Dlog) < G.dh) ++*Dlog;
    return true;
}

// Workspace of the gather: offsets [pairs][Sp+1], ranks [samples], records [samples] (16 B).
struct SortWs {
    long off_bytes, rank_bytes, rec_bytes;
    long total() const { return off_bytes + rank_bytes + rec_bytes; }
};

bool sort_layout(const MsdaGeom& G, MsdaSortCfg* C, SortWs* W)
{
    if (G.dh < 4 || G.dh > 64) return false;
    const long gout_bytes = (long)G.n * G.q * G.m * G.dh * 4;
    if (gout_bytes >= (1L << 31) - 64) return false;
    long Sp = 0;
    for (int l = 0; l < G.L; ++l) {
        C->pstart[l] = (int)Sp;
        Sp += (long)(G.H[l] + 1) * (G.W[l] + 1);
    }
    const long pairs = (long)G.n * G.m;
    if (pairs * (Sp + 1) >= (1L << 31)) return false;
    C->Sp = (int)Sp;
    const int lpc = G.dh / 4;
    long blk = 0;
    for (int k = 0; k < G.L; ++k) {
        const int l = G.L - 1 - k;
        C->blk_start[k] = (int)blk;
        // Records a block of CB cells of this level reads if the samples
        // spread evenly: len_q * points samples per pair land on the level,
        // one record each in a bucket, and a block reads CB+1 of its row's
        // bucket columns in two bucket rows.
        const double expect = 2.0 * G.q * G.P * (CB + 1) / ((double)(G.H[l] + 1) * (G.W[l] + 1));
        int gpc = 1;
        while (gpc < 256 / lpc && expect > 64.0 * gpc) gpc *= 2;   // about 64 records a group
        C->gpc[l] = gpc;
        const int bpw = 256 / (lpc * gpc);   // blocks per workgroup
        const long blocks = (long)G.H[l] * ((G.W[l] + CB - 1) / CB);
        C->wg_per_pair[l] = (int)((blocks + bpw - 1) / bpw);
        blk += (pairs * C->wg_per_pair[l] + 7) & ~7L;
        if (blk >= (1L << 31)) return false;
    }
    C->blk_start[G.L] = (int)blk;
    const long ns = pairs * G.q * G.L * G.P;
    W->off_bytes = (pairs * (Sp + 1) * 4 + 255) & ~255L;
    W->rank_bytes = (ns * 4 + 255) & ~255L;
    W->rec_bytes = ns * 16;
    return true;
}

template <int LPC>
void launch_cells(const MsdaGeom& G, const MsdaSortCfg& C, int LPlog, const int* boff, const int4* rec,
                  const float* gout, float* gvalue, hipStream_t s)
{
    const uint32_t gout_bytes = (uint32_t)((long)G.n * G.q * G.m * G.dh * 4);
    msda_bwd_cells<LPC><<<dim3((unsigned)C.blk_start[G.L]), dim3(256), 0, s>>>(G, C, LPlog, boff, rec, gout,
                                                                               gout_bytes, gvalue);
}

}  // namespace

size_t msda_backward_workspace(const MsdaGeom& G)
{
    MsdaSortCfg C;
    SortWs W;
    int LPlog, Dlog;
    // Alignment of loc does not change the answer here; the launch re-checks it.
    if (!tile_shape(G, nullptr, nullptr, &LPlog, &Dlog) || !sort_layout(G, &C, &W)) return 0;
    return (size_t)W.total();
}

hipError_t launch_msda_backward(const MsdaGeom& G, const float* value, const float* loc, const float* attn,
                                const float* gout, float* gvalue, float* gloc, float* gattn, void* ws,
                                size_t ws_bytes, hipStream_t s)
{
    const long vcount = (long)G.n * G.S * G.m * G.dh;
    const long items = (long)G.n * G.q * G.m;
    const long value_bytes = vcount * 4;
    int LPlog = 0, Dlog = 0;
    MsdaSortCfg C = {};
    SortWs W = {};
    if (tile_shape(G, loc, gloc, &LPlog, &Dlog)) {
        const bool sorted = gvalue && ws && sort_layout(G, &C, &W) && (long)ws_bytes >= W.total() &&
                            (uintptr_t)ws % 16 == 0 && (uintptr_t)gvalue % 16 == 0 && (uintptr_t)gout % 16 == 0;
        int* boff = nullptr;
        int* rank = nullptr;
        int4* rec = nullptr;
        if (sorted) {
            boff = (int*)ws;
            rank = (int*)((char*)ws + W.off_bytes);
            rec = (int4*)((char*)ws + W.off_bytes + W.rank_bytes);
            const long nb = (long)G.n * G.m * (C.Sp + 1);
            fill_zero_f32<<<dim3((unsigned)std::min((nb / 4 + 255) / 256 + 1, 65536L)), dim3(256), 0, s>>>(
                (float*)boff, nb);
            int lds_limit = 65536, num_cus = 256;
            device_limits(&lds_limit, &num_cus);
            const int lds = C.Sp * 4;
            const long chunks = (((long)G.q << LPlog) + CQ_SAMPLES - 1) / CQ_SAMPLES;
            // the packed (bucket, rank) of the LDS count needs Sp < 2^15
            if (C.Sp < (1 << 15) && lds <= std::min(lds_limit, 96 * 1024) && (long)G.n * G.m * chunks < (1L << 31) &&
                hipFuncSetAttribute((const void*)msda_bwd_count_lds, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    lds) == hipSuccess) {
                msda_bwd_count_lds<<<dim3((unsigned)(G.n * G.m * chunks)), dim3(1024), lds, s>>>(
                    G, C, LPlog, (int)chunks, loc, boff, rank);
            } else {
                const long ns = items << LPlog;
                msda_bwd_count<<<dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s>>>(G, C, LPlog, loc, boff,
                                                                                         rank);
            }
            const int scan_lds = (C.Sp + 1) * 4;
            if (scan_lds <= std::min(lds_limit, 128 * 1024) &&
                hipFuncSetAttribute((const void*)msda_bwd_scan<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    scan_lds) == hipSuccess)
                msda_bwd_scan<true><<<dim3((unsigned)(G.n * G.m)), dim3(1024), scan_lds, s>>>(boff, C.Sp + 1);
            else
                msda_bwd_scan<false><<<dim3((unsigned)(G.n * G.m)), dim3(1024), 0, s>>>(boff, C.Sp + 1);
        } else if (gvalue) {
            fill_zero_f32<<<dim3((unsigned)std::min((vcount / 4 + 255) / 256 + 1, 65536L)), dim3(256), 0, s>>>(
                gvalue, vcount);
        }
        const int V = sorted ? 4 : 1;   // the gather needs head_dim >= 4
        const int QT = tile_queries(G, V);
        const int tiles = (G.q + QT - 1) / QT;
        const long nwg = (long)G.n * G.m * tiles;
        const dim3 grid((unsigned)((nwg + 7) & ~7L)), blk((unsigned)(QT * G.dh / V));
        float* gv_tile = sorted ? nullptr : gvalue;
        const size_t lds = (size_t)QT * G.L * G.P * 32;
#define MS_TILE(SM, SO, VV)                                                                                        \
    msda_bwd_tile<SM, SO, VV><<<grid, blk, lds, s>>>(G, LPlog, Dlog, QT, tiles, (int)nwg, (uint32_t)value_bytes, \
                                                     value, loc, attn, gout, gv_tile, gloc, gattn, C, boff, rank, rec)
        if (G.softmax) {
            if (sorted) MS_TILE(true, true, 4);
            else MS_TILE(true, false, 1);
        } else {
            if (sorted) MS_TILE(false, true, 4);
            else MS_TILE(false, false, 1);
        }
#undef MS_TILE
        if (sorted) {
            switch (G.dh / 4) {
            case 1: launch_cells<1>(G, C, LPlog, boff, rec, gout, gvalue, s); break;
            case 2: launch_cells<2>(G, C, LPlog, boff, rec, gout, gvalue, s); break;
            case 4: launch_cells<4>(G, C, LPlog, boff, rec, gout, gvalue, s); break;
            case 8: launch_cells<8>(G, C, LPlog, boff, rec, gout, gvalue, s); break;
            default: launch_cells<16>(G, C, LPlog, boff, rec, gout, gvalue, s); break;
            }
        }
        return hipGetLastError();
    }
    if (gvalue) {
        const long blocks = std::min((vcount / 4 + 255) / 256 + 1, 65536L);
        fill_zero_f32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(gvalue, vcount);
    }
    const dim3 grid((unsigned)((items + 255) / 256));
    if (G.softmax)
        msda_bwd_generic<true><<<grid, dim3(256), 0, s>>>(G, value, loc, attn, gout, gvalue, gloc, gattn);
    else
        msda_bwd_generic<false><<<grid, dim3(256), 0, s>>>(G, value, loc, attn, gout, gvalue, gloc, gattn);
    return hipGetLastError();
}

}  // namespace dcn
