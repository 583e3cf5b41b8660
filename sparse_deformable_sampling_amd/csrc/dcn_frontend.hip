// DCNv4 front-end for gfx950: the offsets and modulation the core op reads,
// produced from the module input x.
//
// "DCNv4: Unbounded Weights", "1. Remove Softmax": with the softmax gone the
// offsets and the modulation come from ONE linear layer, and the offset
// subnetwork is a separable convolution: a depthwise 3x3 convolution, then
// that linear layer (no LayerNorm or GELU between them).  So for every pixel
//   d   = depthwise3x3(x)                       (stride 1, zero padding 1)
//   om  = W_om d + b_om                         (C -> G*K*3 outputs, W_om [G*K*3][C])
//   offset[g][k][0..1] = om[(g*K + k)*2 + 0..1],  mask[g][k] = om[G*K*2 + g*K + k].
//
// The op reads x once and writes G*K*3 values per pixel (more bytes out than
// in for the usual G*K*3 > C): it is HBM-bound; the product is small but
// dense, so it goes on the matrix cores: om^T = W_om d^T with
// v_mfma_f32_16x16x32 (f16 or bf16 operands, fp32 sums), 16 weight rows as
// the A operand and 16 pixels of d as the B operand.  Lane l then holds four
// consecutive outputs of one pixel, which go out as one 8-byte write.  Both
// kernels work on consecutive pixels of the flattened [n][h][w] order, whose
// outputs are one contiguous block of the offset tensor and one of the mask
// tensor: they assemble that block in LDS and write it with 16-byte stores.
//
// Two kernels:
//  - dcn_offset_mask_wave (C up to 256, C/8 dividing 64): W_om in LDS once
//    per workgroup, then each wave alone on its own 16-pixel blocks (see the
//    comment above it);
//  - dcn_offset_mask_k, the tile kernel for the other C: a workgroup of 16
//    waves takes TM = 16, 32 or 64 pixels, computes their depthwise 3x3 (a
//    thread per (pixel, 8 channels), 16-byte loads, fp32 sums, d rounded
//    once to the storage type) into an LDS tile A[TM][C] (rows C+8 elements
//    apart, so that the 16 rows one operand read touches fall on distinct
//    banks), and wave w takes the 16-output blocks w, w+16, ..., reading
//    the weight rows straight from L2 in whole 128-byte lines, one batch
//    ahead of its products.  The kernel waits on memory more than it works
//    (one workgroup per CU at 64-pixel tiles), so it runs as many waves as
//    a workgroup takes: each then walks fewer blocks, whose L2 reads would
//    otherwise wait one after another (stage-3: 4 waves 33.4 us, 8 waves
//    28.8, 16 waves 25.6; whole-line weight reads with batched operand
//    reads 25.0; the first weight batch issued before the depthwise 24.5).
#include <algorithm>

#include "dcn_device.h"
#include "dcn_launch.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr int FT_THREADS = 1024;

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Unsigned division by a runtime constant d >= 1 for n < 2^31 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t m;
    int l;
};

FastDiv make_fastdiv(uint32_t d)
{
    int l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f)
{
    return (__umulhi(n, f.m) + n) >> f.l;
}

struct FrontCfg {
    int KP;          // C rounded up to 32 (the MFMA k extent)
    int AST;         // A tile row stride in elements (KP + 8)
    int NO;          // G*K*3 outputs
    int NOFF;        // G*K*2 of them are offsets
    int ncb;         // 16-output blocks: ceil(NO / 16)
    int npix;        // n * h * w
    int ntiles;
    int o_off;       // byte offset in LDS of the offset image [TM][NOFF]
    int o_mask;      // byte offset in LDS of the mask image [TM][NOFF/2]
    int lds_bytes;
    int mb;          // 16-pixel blocks per tile (TM = 16 * mb)
    int c8;          // 8-channel groups per row of A (KP / 8)
    int dp, dc;      // item step of a thread: FT_THREADS = dp * c8 + dc
    uint32_t x_bytes;
    FastDiv div_w, div_h;
};

// One 16x16x32 product-accumulate; a and b each hold 8 storage-type values
// (lane l: row of a / column of b l%16, k block l/16).
template <int DT>
__device__ __forceinline__ f4_t mfma32(uint4 a, uint4 b, f4_t c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c, 0, 0,
                                                      0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c, 0,
                                                       0, 0);
}

// Widen 8 storage-type values held in a 16-byte register to fp32.
template <int DT>
__device__ __forceinline__ void widen8(u32x4 r, float* v)
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (DT == DT_F16) {
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        } else {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// Two storage-type values packed into one dword (first in the low half).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return pack2_rne<DT>(a, b);
}

// Copy `bytes` (even) bytes from LDS to global memory: 16 bytes per thread and
// step, then the 2-byte tail.  Both starts are 16-byte aligned.
__device__ __forceinline__ void copy_out(const unsigned char* src, unsigned char* dst, int bytes, int tid)
{
    const int nv = bytes >> 4;
    for (int u = tid; u < nv; u += FT_THREADS) {
        *reinterpret_cast<uint4*>(dst + (size_t)u * 16) = *reinterpret_cast<const uint4*>(src + u * 16);
        count_writes(dst + (size_t)u * 16, 8);
    }
    const int tail = (bytes - nv * 16) >> 1;
    if (tid < tail) {
        *reinterpret_cast<uint16_t*>(dst + (size_t)nv * 16 + tid * 2) =
            *reinterpret_cast<const uint16_t*>(src + nv * 16 + tid * 2);
        count_writes(dst + (size_t)nv * 16 + tid * 2, 1);
    }
}

template <int DT, int MB>
__global__ __launch_bounds__(FT_THREADS) void dcn_offset_mask_k(Geom G, FrontCfg F,
                                                               const typename Elem<DT>::T* __restrict__ x,
                                                               const typename Elem<DT>::T* __restrict__ dww,
                                                               const typename Elem<DT>::T* __restrict__ dwb,
                                                               const typename Elem<DT>::T* __restrict__ omw,
                                                               const typename Elem<DT>::T* __restrict__ omb,
                                                               typename Elem<DT>::T* __restrict__ off,
                                                               typename Elem<DT>::T* __restrict__ mask)
{
    using T = typename Elem<DT>::T;
    constexpr int TM = 16 * MB;
    extern __shared__ __align__(16) unsigned char lds[];
    T* A = reinterpret_cast<T*>(lds);                  // [TM][AST]
    T* Ooff = reinterpret_cast<T*>(lds + F.o_off);     // [TM][NOFF]
    T* Omask = reinterpret_cast<T*>(lds + F.o_mask);   // [TM][NOFF/2]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = G.c, H = G.h, W = G.w;
    const int NOFF = F.NOFF, NMASK = F.NOFF / 2;
    // Workgroups are dealt to the eight XCDs round-robin; give each XCD a
    // contiguous range of tiles so that the rows above and below a tile, read
    // by its neighbours, are in the same L2.
    const int q8 = F.ntiles / 8, r8 = F.ntiles % 8, xcd = blockIdx.x % 8;
    const int tile = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    const int px0 = tile * TM;
    const int npx = min(TM, F.npix - px0);

    // ---- weight stream set-up (see the product below)
    const int kg = 8 * (lane >> 4);
    const bool quad = (NMASK & 3) == 0;   // 4 consecutive outputs of a pixel are 8-byte aligned in LDS
    const int prow = lane & 7, pchunk = (lane >> 4) + ((lane >> 1) & 4);
    const bool hi8 = (lane & 8) != 0;
    constexpr int FP = (DT == DT_BF16 && MB == 4) ? 2 : 3;          // k-step pairs per batch (3 spill at bf16 64-pixel tiles)
    const int nkb = (F.KP + 64 * FP - 1) / (64 * FP);              // batches per block
    constexpr int NWV = FT_THREADS / 64;
    const int nblk = wave < F.ncb ? (F.ncb - wave + NWV - 1) / NWV : 0;
    const int nit = nblk * nkb;
    auto load_batch = [&](int it, uint4* w, uint32_t* bias) {
        const int j = it / nkb, kb = it - j * nkb;
        const int cb = wave + NWV * j, kc = 64 * FP * kb;
        const T* r0 = omw + (long)min(cb * 16 + prow, F.NO - 1) * C;       // rows past NO compute a copy, not stored
        const T* r1 = omw + (long)min(cb * 16 + 8 + prow, F.NO - 1) * C;
#pragma unroll
        for (int t = 0; t < FP; ++t) {
            const int k0 = kc + 64 * t + 8 * pchunk;
            w[2 * t] = k0 < C ? *reinterpret_cast<const uint4*>(r0 + k0) : make_uint4(0u, 0u, 0u, 0u);
            w[2 * t + 1] = k0 < C ? *reinterpret_cast<const uint4*>(r1 + k0) : make_uint4(0u, 0u, 0u, 0u);
        }
        if (kb == 0) {
            const int j0 = cb * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) bias[i] = __builtin_bit_cast(uint16_t, omb[min(j0 + i, F.NO - 1)]);
        }
    };
    uint4 wcur[2 * FP], wnxt[2 * FP];
    uint32_t bcur[4] = {0u, 0u, 0u, 0u}, bnxt[4] = {0u, 0u, 0u, 0u};   // raw bias bits, widened when used
    f4_t acc[MB];
    // The first batch of this wave's weights does not depend on the tile:
    // it is in flight during the depthwise phase.
    if (nit > 0) load_batch(0, wcur, bcur);

    // ---- depthwise 3x3 into A.  A thread's items are (pixel p, channels
    // 8*cg..) for e = tid, tid + FT_THREADS, ...; rows past the last pixel and
    // channels past C are written as zeros.  A neighbour outside the image
    // reads through an out-of-range buffer offset, which returns zeros.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)F.x_bytes, 0x00020000);
    const uint32_t colB = (uint32_t)C * 2u, rowB = (uint32_t)W * colB;
    int p = tid / F.c8, cg = tid - p * F.c8;
#pragma unroll 2
    for (; p < TM; p += F.dp) {
        const int cc = cg * 8;
        float acc[8];
        if (p < npx && cc < C) {
            const uint32_t pix = (uint32_t)(px0 + p);
            const uint32_t ny = fdiv(pix, F.div_w), xc = pix - ny * (uint32_t)W;
            const uint32_t y = ny - fdiv(ny, F.div_h) * (uint32_t)H;
            const uint32_t base = pix * colB + (uint32_t)cc * 2u;
            const bool up = y > 0, down = y + 1 < (uint32_t)H, left = xc > 0, right = xc + 1 < (uint32_t)W;
            load_vec<DT>(dwb + cc, acc);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const bool ok = (i != 0 || up) && (i != 2 || down) && (j != 0 || left) && (j != 2 || right);
                    const uint32_t o = ok ? base + (uint32_t)(i - 1) * rowB + (uint32_t)(j - 1) * colB : 0x80000000u;
                    float xv[8], wv[8];
                    widen8<DT>(__builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0), xv);
                    load_vec<DT>(dww + (i * 3 + j) * C + cc, wv);
#pragma unroll
                    for (int u = 0; u < 8; ++u) acc[u] = fmaf(wv[u], xv[u], acc[u]);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] = 0.f;
        }
        store_vec<DT>(A + p * F.AST + cc, acc);
        cg += F.dc;
        if (cg >= F.c8) {
            cg -= F.c8;
            ++p;
        }
    }
    __syncthreads();

    // ---- NO x TM product om^T = W_om d^T: wave w takes output blocks w,
    // w+NWV, ... (NWV waves); the A operand is 16 weight rows, the B operand 16 pixels of
    // d.  Lane l then holds outputs j0..j0+3 (j0 = 16*cb + 4*(l/16)) of pixel
    // 16*rb + l%16.
    //
    // Weight rows come from L2 two k steps (64 channels, one 128-byte line of
    // a row) at a time: load i of a pair reads rows 8i..8i+7 of the block in
    // full lines (lane l: row 8i + l%8, 16-byte chunk l/16 + 4*((l/8)%2)),
    // 8 line lookups per KB where the operand layout (16 rows x 64 bytes)
    // would touch 16.  A rotation by 8 lanes within each row of 16 (DPP
    // row_ror) and a select then give each lane its operand chunk: row l%16,
    // chunk l/16 of the pair's first step and 4 + l/16 of its second.  A
    // wave's loads run one batch (FP pairs) ahead of its products, across
    // its blocks, and each block's bias comes with the block's first batch.
    auto ror8 = [](uint4 v) {
        return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x128, 0xF, 0xF, false),
                          (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x128, 0xF, 0xF, false),
                          (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, 0x128, 0xF, 0xF, false),
                          (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, 0x128, 0xF, 0xF, false));
    };
    auto sel = [](bool c, uint4 a, uint4 b) {
        return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
    };
    for (int it = 0; it < nit; ++it) {
        const int j = it / nkb, kb = it - j * nkb;
        const int cb = wave + NWV * j, kc = 64 * FP * kb;
        if (it + 1 < nit) load_batch(it + 1, wnxt, bnxt);
        if (kb == 0) {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) acc[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < FP; ++t) {
            if (kc + 64 * t >= F.KP) break;
            const uint4 e = sel(hi8, ror8(wcur[2 * t + 1]), wcur[2 * t]);
            const uint4 o = sel(hi8, wcur[2 * t + 1], ror8(wcur[2 * t]));
            const int k0 = kc + 64 * t + kg;
            // A step's MB operand reads are issued together, ahead of its
            // products, so that their LDS latency is paid once per step.
            uint4 bf[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) bf[rb] = *reinterpret_cast<const uint4*>(A + (rb * 16 + (lane & 15)) * F.AST + k0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) acc[rb] = mfma32<DT>(e, bf[rb], acc[rb]);
            if (kc + 64 * t + 32 < F.KP) {
#pragma unroll
                for (int rb = 0; rb < MB; ++rb)
                    bf[rb] = *reinterpret_cast<const uint4*>(A + (rb * 16 + (lane & 15)) * F.AST + k0 + 32);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rb = 0; rb < MB; ++rb) acc[rb] = mfma32<DT>(o, bf[rb], acc[rb]);
            }
        }
        if (kb == nkb - 1) {
            const int j0 = cb * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) {
                const int row = rb * 16 + (lane & 15);
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = acc[rb][i] + to_f32(__builtin_bit_cast(T, (uint16_t)bcur[i]));
                if (quad && j0 + 3 < NOFF) {
                    *reinterpret_cast<uint2*>(Ooff + row * NOFF + j0) = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
                } else if (quad && j0 >= NOFF && j0 + 3 < F.NO) {
                    *reinterpret_cast<uint2*>(Omask + row * NMASK + (j0 - NOFF)) =
                        make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int jj = j0 + i;
                        if (jj < NOFF) Ooff[row * NOFF + jj] = from_f32<DT>(v[i]);
                        else if (jj < F.NO) Omask[row * NMASK + (jj - NOFF)] = from_f32<DT>(v[i]);
                    }
                }
            }
        }
        if (it + 1 < nit) {
#pragma unroll
            for (int i = 0; i < 2 * FP; ++i) wcur[i] = wnxt[i];
            if ((it + 1) % nkb == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) bcur[i] = bnxt[i];
            }
        }
    }
    __syncthreads();

    // ---- the tile's outputs are contiguous in both tensors
    copy_out(lds + F.o_off, reinterpret_cast<unsigned char*>(off + (long)px0 * NOFF), npx * NOFF * 2, tid);
    copy_out(lds + F.o_mask, reinterpret_cast<unsigned char*>(mask + (long)px0 * NMASK), npx * NMASK * 2, tid);
}

// ---------------------------------------------------------------------------
// Wave-independent kernel for C8 = KP/8 in {4, 8, 16, 32} (C up to 256): the
// weights W_om (zero-padded to 16-row blocks) and the bias are loaded into
// LDS once per workgroup; after that every wave works on its own 16-pixel
// blocks with no workgroup barrier, so that waves in different phases
// (loads, products, stores) overlap on a CU.  A lane keeps one 8-channel
// group (lane % C8) for good, with its nine depthwise weight vectors and
// bias in registers, and slides a 3 x (R+2) window of x along a run of R
// pixels of one image row (R = 2 for even widths: six 16-byte loads per
// pixel instead of nine).  The wave's d tile [16][KP] sits in its own LDS
// slice; once its MFMA operands are in registers, the block's output image
// takes the same bytes.

struct WaveCfg {
    int AST;         // A / Bt row stride in elements (KP + 8)
    int NO, NOFF;    // G*K*3 outputs, G*K*2 of them offsets
    int ncb;         // 16-output blocks
    int npix, nblk;  // pixels, 16-pixel blocks
    int nw;          // waves per workgroup (4 or 8, or 9-16 for one block per wave; chosen at launch)
    int nwg;         // workgroups, a multiple of 8 (chosen at launch)
    int bias_off;    // LDS byte offsets: Bt at 0, bias (fp32), wave slices
    int dw_off;      // bf16 only: depthwise weights [9][KP] and bias [KP] as fp32
    int w_off, w_bytes;  // wave slices: A [16][AST], then the output image in the same bytes
    int lds_bytes;   // w_off + nw * w_bytes
    uint32_t x_bytes;
    FastDiv div_w, div_h;
};

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// acc[u] += w[u] * x[u] for 8 storage-type values in each of w and x.
template <int DT>
__device__ __forceinline__ void fma8(u32x4 w, u32x4 x, float* acc)
{
    float wv[8], xv[8];
    widen8<DT>(w, wv);
    widen8<DT>(x, xv);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = fmaf(wv[u], xv[u], acc[u]);
}

__device__ __forceinline__ void wave_copy_out(const unsigned char* src, unsigned char* dst, int bytes, int lane)
{
    const int nv = bytes >> 4;
    for (int u = lane; u < nv; u += 64) {
        *reinterpret_cast<uint4*>(dst + (size_t)u * 16) = *reinterpret_cast<const uint4*>(src + u * 16);
        count_writes(dst + (size_t)u * 16, 8);
    }
    const int tail = (bytes - nv * 16) >> 1;
    if (lane < tail) {
        *reinterpret_cast<uint16_t*>(dst + (size_t)nv * 16 + lane * 2) =
            *reinterpret_cast<const uint16_t*>(src + nv * 16 + lane * 2);
        count_writes(dst + (size_t)nv * 16 + lane * 2, 1);
    }
}

template <int DT, int C8, int R, int NWMAX>
__global__ __launch_bounds__(NWMAX * 64) void dcn_offset_mask_wave(Geom G, WaveCfg F, const typename Elem<DT>::T* __restrict__ x,
                                                             const typename Elem<DT>::T* __restrict__ dww,
                                                             const typename Elem<DT>::T* __restrict__ dwb,
                                                             const typename Elem<DT>::T* __restrict__ omw,
                                                             const typename Elem<DT>::T* __restrict__ omb,
                                                             typename Elem<DT>::T* __restrict__ off,
                                                             typename Elem<DT>::T* __restrict__ mask)
{
    using T = typename Elem<DT>::T;
    constexpr int KP = C8 * 8, KS = KP / 32;       // MFMA k steps
    constexpr int RUNS = 16 / R;                  // runs per block
    constexpr int LPR = 64 / C8;                  // runs one pass of the wave covers
    extern __shared__ __align__(16) unsigned char lds[];
    T* Bt = reinterpret_cast<T*>(lds);                           // [ncb*16][AST]
    const float* bs = reinterpret_cast<const float*>(lds + F.bias_off);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int C = G.c, H = G.h, W = G.w;
    const int AST = F.AST, NOFF = F.NOFF, NMASK = F.NOFF / 2, NO = F.NO;

    // ---- once per workgroup: W_om rows (zero past NO and C) and the bias
    {
        float* bsw = reinterpret_cast<float*>(lds + F.bias_off);
        const int nthr = F.nw * 64;
        for (int e = tid; e < F.ncb * 16 * C8; e += nthr) {
            const int j = e / C8, k8 = (e - j * C8) * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (j < NO && k8 < C) v = *reinterpret_cast<const uint4*>(omw + (long)j * C + k8);
            *reinterpret_cast<uint4*>(Bt + j * AST + k8) = v;
        }
        for (int j = tid; j < NO; j += nthr) bsw[j] = to_f32(omb[j]);
        if constexpr (DT == DT_BF16) {
            // bf16 has no mixed-precision multiply-add: the depthwise weights and
            // bias are widened once here instead of at every use
            float* dwf = reinterpret_cast<float*>(lds + F.dw_off);
            for (int e = tid; e < 10 * KP; e += nthr) {
                const int t = e / KP, c = e - t * KP;
                dwf[e] = c >= C ? 0.f : to_f32(t < 9 ? dww[t * C + c] : dwb[c]);
            }
        }
    }
    __syncthreads();

    unsigned char* slice = lds + F.w_off + wid * F.w_bytes;
    T* A = reinterpret_cast<T*>(slice);                           // [16][AST]
    T* Ooff = reinterpret_cast<T*>(slice);                        // [16][NOFF], over A once it is read
    T* Omask = Ooff + 16 * NOFF;                                  // [16][NMASK]

    // this lane's channel group, its depthwise weights and bias
    const int cc = (lane % C8) * 8;
    const bool live = cc < C;
    u32x4 wr[9], br = u32x4{0u, 0u, 0u, 0u};
    if constexpr (DT != DT_BF16) {
#pragma unroll
        for (int t = 0; t < 9; ++t)
            wr[t] = live ? *reinterpret_cast<const u32x4*>(dww + t * C + cc) : u32x4{0u, 0u, 0u, 0u};
        if (live) br = *reinterpret_cast<const u32x4*>(dwb + cc);
    }
    const float* dwf = reinterpret_cast<const float*>(lds + F.dw_off) + cc;   // bf16: [t][KP], bias at t = 9

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)F.x_bytes, 0x00020000);
    const uint32_t colB = (uint32_t)C * 2u, rowB = (uint32_t)W * colB;
    const int kg = 8 * (lane >> 4);
    const bool quad = (NMASK & 3) == 0;

    // blocks: each XCD sweeps a contiguous range, its waves interleaved
    const int xcd = blockIdx.x % 8, nwx = (gridDim.x / 8) * F.nw;
    const int q8 = F.nblk / 8, r8 = F.nblk % 8;
    const int lo = xcd * q8 + min(xcd, r8), cnt = q8 + (xcd < r8 ? 1 : 0);
    for (int bi = (blockIdx.x / 8) * F.nw + wid; bi < cnt; bi += nwx) {
        const int px0 = (lo + bi) * 16;
        const int npx = min(16, F.npix - px0);

        // ---- depthwise into A: runs lane/C8, lane/C8 + LPR, ...  With R = 2
        // the width is even, so a run never leaves its image row and a run
        // that starts on a pixel ends on one.  Rows past the block's pixels
        // are left as they are: they only feed output columns that are not
        // stored.  Channel groups past C are written as zeros.
#pragma unroll 1
        for (int ru = lane / C8; ru < RUNS; ru += LPR) {
            const int p0 = ru * R;
            if (p0 >= npx) continue;
            // keep the weights packed from run to run: their widening stays at
            // the point of use instead of being hoisted into 72 live registers
            if constexpr (DT != DT_BF16) {
#pragma unroll
                for (int t = 0; t < 9; ++t) asm volatile("" : "+v"(wr[t].x), "+v"(wr[t].y), "+v"(wr[t].z), "+v"(wr[t].w));
                asm volatile("" : "+v"(br.x), "+v"(br.y), "+v"(br.z), "+v"(br.w));
            }
            float acc[R][8];
            if (live) {
                const uint32_t pix0 = (uint32_t)(px0 + p0);
                const uint32_t ny = fdiv(pix0, F.div_w), xc = pix0 - ny * (uint32_t)W;
                const uint32_t y = ny - fdiv(ny, F.div_h) * (uint32_t)H;
                const uint32_t base = pix0 * colB + (uint32_t)cc * 2u;
                const bool up = y > 0, down = y + 1 < (uint32_t)H, left = xc > 0, right = xc + R < (uint32_t)W;
                u32x4 X[3][R + 2];
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < R + 2; ++j) {
                        const bool ok = (i != 0 || up) && (i != 2 || down) && (j != 0 || left) && (j != R + 1 || right);
                        const uint32_t o =
                            ok ? base + (uint32_t)(i - 1) * rowB + (uint32_t)(j - 1) * colB : 0x80000000u;
                        X[i][j] = __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0);
                    }
                if constexpr (DT == DT_BF16) {
                    float xv[3][R + 2][8];
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int j = 0; j < R + 2; ++j) widen8<DT>(X[i][j], xv[i][j]);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float4 b0 = *reinterpret_cast<const float4*>(dwf + 9 * KP);
                        const float4 b1 = *reinterpret_cast<const float4*>(dwf + 9 * KP + 4);
                        acc[r][0] = b0.x; acc[r][1] = b0.y; acc[r][2] = b0.z; acc[r][3] = b0.w;
                        acc[r][4] = b1.x; acc[r][5] = b1.y; acc[r][6] = b1.z; acc[r][7] = b1.w;
                    }
#pragma unroll
                    for (int t = 0; t < 9; ++t) {
                        const int i = t / 3, j = t % 3;
                        const float4 w0 = *reinterpret_cast<const float4*>(dwf + t * KP);
                        const float4 w1 = *reinterpret_cast<const float4*>(dwf + t * KP + 4);
                        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int u = 0; u < 8; ++u) acc[r][u] = fmaf(wv[u], xv[i][r + j][u], acc[r][u]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        widen8<DT>(br, acc[r]);
#pragma unroll
                        for (int i = 0; i < 3; ++i)
#pragma unroll
                            for (int j = 0; j < 3; ++j) fma8<DT>(wr[i * 3 + j], X[i][r + j], acc[r]);
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int u = 0; u < 8; ++u) acc[r][u] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) store_vec<DT>(A + (p0 + r) * AST + cc, acc[r]);
        }
        wave_lds_sync();

        // ---- om^T = W_om d^T for the block's 16 pixels: d fragments held in
        // registers, weight fragments read from LDS; lane l ends with outputs
        // j0..j0+3 (j0 = 16*cb + 4*(l/16)) of pixel l%16.
        uint4 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) af[ks] = *reinterpret_cast<const uint4*>(A + (lane & 15) * AST + ks * 32 + kg);
        wave_lds_sync();   // A is in registers now; the output image overwrites it
        const int row = lane & 15;
#pragma unroll 2
        for (int cb = 0; cb < F.ncb; ++cb) {
            const T* bp = Bt + (cb * 16 + (lane & 15)) * AST + kg;
            f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma32<DT>(*reinterpret_cast<const uint4*>(bp + ks * 32), af[ks], acc);
            const int j0 = cb * 16 + 4 * (lane >> 4);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[i] + bs[min(j0 + i, NO - 1)];
            if (quad && j0 + 3 < NOFF) {
                *reinterpret_cast<uint2*>(Ooff + row * NOFF + j0) = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
            } else if (quad && j0 >= NOFF && j0 + 3 < NO) {
                *reinterpret_cast<uint2*>(Omask + row * NMASK + (j0 - NOFF)) =
                    make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = j0 + i;
                    if (j < NOFF) Ooff[row * NOFF + j] = from_f32<DT>(v[i]);
                    else if (j < NO) Omask[row * NMASK + (j - NOFF)] = from_f32<DT>(v[i]);
                }
            }
        }
        wave_lds_sync();

        // ---- the block's outputs are contiguous in both tensors
        wave_copy_out(reinterpret_cast<const unsigned char*>(Ooff), reinterpret_cast<unsigned char*>(off + (long)px0 * NOFF),
                      npx * NOFF * 2, lane);
        wave_copy_out(reinterpret_cast<const unsigned char*>(Omask),
                      reinterpret_cast<unsigned char*>(mask + (long)px0 * NMASK), npx * NMASK * 2, lane);
        wave_lds_sync();   // the image is read out before the next block rewrites it
    }
}

template <int DT, int C8, int R>
hipError_t launch_wave_c8(const Geom& G, const WaveCfg& F, const void* x, const void* dww, const void* dwb,
                          const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    // Where 8-wave workgroups would leave some waves two blocks and others
    // one (between 8 and 16 blocks per CU), one workgroup per CU with a wave
    // for each block, up to 16 waves (one-pixel runs, <= 128 registers),
    // ends every wave after one block (stage-2, 28x28x128: f16 22.2 ->
    // 20.2 us, bf16 29.8 -> 24.3 us).
    {
        int lds_limit, num_cus;
        device_limits(&lds_limit, &num_cus);
        const int nw1 = (F.nblk + num_cus - 1) / num_cus;
        if (R == 1 && nw1 > 8 && nw1 <= 16 && F.w_off + nw1 * F.w_bytes <= lds_limit) {
            auto* fb = dcn_offset_mask_wave<DT, C8, 1, 16>;
            WaveCfg L = F;
            L.nw = nw1;
            L.lds_bytes = F.w_off + nw1 * F.w_bytes;
            hipError_t e = hipFuncSetAttribute((const void*)fb, hipFuncAttributeMaxDynamicSharedMemorySize, L.lds_bytes);
            if (e != hipSuccess) return e;
            int per_cu = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fb, nw1 * 64, L.lds_bytes);
            if (e != hipSuccess) return e;
            if (per_cu >= 1) {
                L.nwg = (std::min((F.nblk + nw1 - 1) / nw1, num_cus) + 7) / 8 * 8;
                fb<<<dim3(L.nwg), dim3(nw1 * 64), L.lds_bytes, s>>>(G, L, (const T*)x, (const T*)dww, (const T*)dwb,
                                                                  (const T*)omw, (const T*)omb, (T*)off, (T*)mask);
                return hipGetLastError();
            }
        }
    }
    auto* fn = dcn_offset_mask_wave<DT, C8, R, 8>;
    // Workgroups of 4 or 8 waves, whichever keeps more waves resident on a
    // CU (the weights are loaded once per workgroup: ties go to 8); as many
    // workgroups as stay resident together, a multiple of 8 (one range of
    // blocks per XCD).
    int lds_limit, num_cus;
    device_limits(&lds_limit, &num_cus);
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       std::min(F.w_off + 8 * F.w_bytes, lds_limit));
    if (e != hipSuccess) return e;
    WaveCfg L = F;
    int best = -1;
    for (int nw = 8; nw >= 4; nw /= 2) {
        const int bytes = F.w_off + nw * F.w_bytes;
        if (bytes > lds_limit) continue;
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, nw * 64, bytes);
        if (e != hipSuccess) return e;
        if (per_cu * nw > best) {
            best = per_cu * nw;
            L.nw = nw;
            L.lds_bytes = bytes;
        }
    }
    if (best < 0) return hipErrorInvalidValue;
    const int need = (F.nblk + L.nw - 1) / L.nw;
    L.nwg = (std::min(need, std::max(1, best / L.nw) * num_cus) + 7) / 8 * 8;
    fn<<<dim3(L.nwg), dim3(L.nw * 64), L.lds_bytes, s>>>(G, L, (const T*)x, (const T*)dww, (const T*)dwb,
                                                         (const T*)omw, (const T*)omb, (T*)off, (T*)mask);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_wave(const Geom& G, const WaveCfg& F, int c8, const void* x, const void* dww, const void* dwb,
                       const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    // Runs of two pixels need an even width.  bf16 keeps its whole widened
    // 3x4 window live (96 registers); from 128 channels on one-pixel runs
    // leave room for more waves (Table 10 shape: 55 -> 46 us).  The
    // one-block-per-wave launch (see launch_wave_c8) takes one-pixel runs.
    int lds_limit, num_cus;
    device_limits(&lds_limit, &num_cus);
    const int nw1 = (F.nblk + num_cus - 1) / num_cus;
    const bool one = nw1 > 8 && nw1 <= 16 && F.w_off + nw1 * F.w_bytes <= lds_limit;
    const bool r2 = !one && G.w % 2 == 0 && !(DT == DT_BF16 && c8 >= 16);
#define DCN_FE_CASE(N)                                                                          \
    case N:                                                                                     \
        return r2 ? launch_wave_c8<DT, N, 2>(G, F, x, dww, dwb, omw, omb, off, mask, s)        \
                  : launch_wave_c8<DT, N, 1>(G, F, x, dww, dwb, omw, omb, off, mask, s);
    switch (c8) {
        DCN_FE_CASE(4)
        DCN_FE_CASE(8)
        DCN_FE_CASE(16)
        DCN_FE_CASE(32)
    }
#undef DCN_FE_CASE
    return hipErrorInvalidValue;
}

// Plan of the wave kernel; false (use the tile kernel) when C rounded up to
// 32 is not 32, 64, 128 or 256 or the weights and 4 wave slices exceed LDS.
bool plan_wave(const Geom& G, int dtype, int lds_limit, int num_cus, WaveCfg* F, int* c8)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    if (G.c % 8 != 0) return false;
    if ((long)G.n * G.h * G.w * G.c * 2 >= (1l << 31)) return false;
    const int KP = (G.c + 31) / 32 * 32;
    if (KP != 32 && KP != 64 && KP != 128 && KP != 256) return false;
    *c8 = KP / 8;
    F->AST = KP + 8;
    F->NO = G.g * G.K * 3;
    F->NOFF = G.g * G.K * 2;
    F->ncb = (F->NO + 15) / 16;
    F->npix = G.n * G.h * G.w;
    F->nblk = (F->npix + 15) / 16;
    const int b_bytes = F->ncb * 16 * F->AST * 2;
    F->bias_off = b_bytes;
    F->dw_off = (b_bytes + F->NO * 4 + 15) / 16 * 16;
    F->w_off = F->dw_off + (dtype == DT_BF16 ? 10 * KP * 4 : 0);
    F->w_bytes = std::max(16 * F->AST * 2, 48 * F->NOFF);
    // workgroup size and count are set at launch from the kernel's occupancy
    F->nw = 4;
    F->lds_bytes = F->w_off + F->nw * F->w_bytes;
    if (F->lds_bytes > lds_limit) return false;
    F->nwg = 0;
    F->x_bytes = (uint32_t)((long)G.n * G.h * G.w * G.c * 2);
    F->div_w = make_fastdiv((uint32_t)G.w);
    F->div_h = make_fastdiv((uint32_t)G.h);
    return true;
}

template <int DT, int MB>
hipError_t launch_mb(const Geom& G, const FrontCfg& F, const void* x, const void* dww, const void* dwb,
                     const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    auto* fn = dcn_offset_mask_k<DT, MB>;
    const hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, F.lds_bytes);
    if (e != hipSuccess) return e;
    fn<<<dim3(F.ntiles), dim3(FT_THREADS), F.lds_bytes, s>>>(G, F, (const T*)x, (const T*)dww, (const T*)dwb,
                                                            (const T*)omw, (const T*)omb, (T*)off, (T*)mask);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_typed(const Geom& G, const FrontCfg& F, const void* x, const void* dww, const void* dwb,
                        const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    switch (F.mb) {
    case 4: return launch_mb<DT, 4>(G, F, x, dww, dwb, omw, omb, off, mask, s);
    case 2: return launch_mb<DT, 2>(G, F, x, dww, dwb, omw, omb, off, mask, s);
    default: return launch_mb<DT, 1>(G, F, x, dww, dwb, omw, omb, off, mask, s);
    }
}

void layout(const Geom& G, int mb, FrontCfg* F)
{
    const int tm = 16 * mb;
    F->mb = mb;
    F->KP = (G.c + 31) / 32 * 32;
    F->AST = F->KP + 8;
    F->NO = G.g * G.K * 3;
    F->NOFF = G.g * G.K * 2;
    F->ncb = (F->NO + 15) / 16;
    F->npix = G.n * G.h * G.w;
    F->ntiles = (F->npix + tm - 1) / tm;
    F->o_off = tm * F->AST * 2;
    F->o_mask = F->o_off + tm * F->NOFF * 2;
    F->lds_bytes = F->o_mask + tm * F->NOFF;
    F->c8 = F->KP / 8;
    F->dp = FT_THREADS / F->c8;
    F->dc = FT_THREADS % F->c8;
    F->x_bytes = (uint32_t)((long)G.n * G.h * G.w * G.c * 2);
    F->div_w = make_fastdiv((uint32_t)G.w);
    F->div_h = make_fastdiv((uint32_t)G.h);
}

// Tile plan.  Every tile streams all of W_om from L2, so per CU the cost is
// about (tiles per CU) x (W_om's lines + the tile's own depthwise reads and
// output lines), the weights counted at 16 lookups per KB of the operand
// layout (the load order reads whole lines, 8 per KB, but the stream's
// latency scales the same way).  Take the tile size that fits in LDS with
// the least such cost (ties to the larger tile).  At stage-3 (320 channels,
// 540 outputs) 64-pixel tiles, one 16-wave workgroup per CU, take 25.0 us
// against 35.4 for 32-pixel tiles and 33.6 for 32-pixel tiles in 8-wave
// workgroups two per CU: the time grows with the number of tiles, each of
// which streams the 346 KB of weights.  False if not even a 16-pixel tile
// fits.
bool plan_frontend(const Geom& G, int dtype, int lds_limit, int num_cus, FrontCfg* F)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    if (G.c % 8 != 0) return false;
    if ((long)G.n * G.h * G.w * G.c * 2 >= (1l << 31)) return false;   // buffer offsets, out-of-range marker 2^31
    int best = 0;
    double best_cost = 0.0;
    for (int mb = 4; mb >= 1; mb /= 2) {
        layout(G, mb, F);
        if (F->lds_bytes > lds_limit) continue;
        const double w_lines = (double)F->ncb * (F->KP / 32) * 16;
        const double px_lines = 9.0 * G.c * 2 / 128 + (double)F->NO * 2 / 128;
        const double cost = (double)((F->ntiles + num_cus - 1) / num_cus) * (w_lines + 16.0 * mb * px_lines);
        if (best == 0 || cost < best_cost) {
            best = mb;
            best_cost = cost;
        }
    }
    if (best == 0) return false;
    layout(G, best, F);
    return true;
}

}  // namespace

bool frontend_supported(const Geom& G, int dtype, int lds_limit)
{
    FrontCfg F;
    return plan_frontend(G, dtype, lds_limit, 1, &F);
}

hipError_t launch_dcn_offset_mask(const Geom& G, int dtype, const void* x, const void* dww, const void* dwb,
                                  const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    int lds_limit, num_cus;
    device_limits(&lds_limit, &num_cus);
    WaveCfg WF;
    int c8;
    if (plan_wave(G, dtype, lds_limit, num_cus, &WF, &c8))
        return dtype == DT_F16 ? launch_wave<DT_F16>(G, WF, c8, x, dww, dwb, omw, omb, off, mask, s)
                               : launch_wave<DT_BF16>(G, WF, c8, x, dww, dwb, omw, omb, off, mask, s);
    FrontCfg F;
    if (!plan_frontend(G, dtype, lds_limit, num_cus, &F)) return hipErrorInvalidValue;
    return dtype == DT_F16 ? launch_typed<DT_F16>(G, F, x, dww, dwb, omw, omb, off, mask, s)
                           : launch_typed<DT_BF16>(G, F, x, dww, dwb, omw, omb, off, mask, s);
}

#ifdef DCN_COUNT_WRITES
DCN_WRITE_COUNT_SETTER(frontend_count_writes)
#endif

}  // namespace dcn
