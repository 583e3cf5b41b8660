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
// in for the usual G*K*3 > C): it is HBM-bound, the product is small.  One
// workgroup of four waves takes a tile of TM consecutive pixels in the
// flattened [n][h][w] order (no idle rows at narrow maps):
//  - depthwise: a thread takes (pixel, 8 channels), reads the 3x3
//    neighbourhood with 16-byte loads (the overlapping rows hit in cache),
//    sums in fp32 and writes d, rounded once to the storage type, into an LDS
//    tile A[TM][C] (row stride C+8 elements, so that the 16 rows one MFMA
//    operand read touches fall on distinct banks);
//  - the linear layer on the matrix cores, v_mfma_f32_16x16x32 (f16 or bf16
//    operands, fp32 sums): wave w takes 16-column blocks w, w+4, ...; the A
//    operand comes from LDS, the B operand straight from W_om in global memory
//    (16 contiguous bytes of one weight row per lane; the weights, a few KB to
//    a few hundred KB, stay in L2 across workgroups);
//  - epilogue: bias added in fp32, each value rounded once into an LDS image
//    of the tile's outputs.  For consecutive pixels these are one contiguous
//    block of the offset tensor and one of the mask tensor, which the
//    workgroup then writes with 16-byte stores.
#include <algorithm>

#include "dcn_device.h"
#include "dcn_launch.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr int FT_THREADS = 256;
constexpr int FT_LDS_TARGET = 80 * 1024;   // two workgroups per CU

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
    int dp, dc;      // item step of a thread: 256 = dp * c8 + dc
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
    return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<DT>(a)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<DT>(b)) << 16);
}

// Copy `bytes` (even) bytes from LDS to global memory: 16 bytes per thread and
// step, then the 2-byte tail.  Both starts are 16-byte aligned.
__device__ __forceinline__ void copy_out(const unsigned char* src, unsigned char* dst, int bytes, int tid)
{
    const int nv = bytes >> 4;
    for (int u = tid; u < nv; u += FT_THREADS)
        *reinterpret_cast<uint4*>(dst + (size_t)u * 16) = *reinterpret_cast<const uint4*>(src + u * 16);
    const int tail = (bytes - nv * 16) >> 1;
    if (tid < tail)
        *reinterpret_cast<uint16_t*>(dst + (size_t)nv * 16 + tid * 2) =
            *reinterpret_cast<const uint16_t*>(src + nv * 16 + tid * 2);
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

    // ---- depthwise 3x3 into A.  A thread's items are (pixel p, channels
    // 8*cg..) for e = tid, tid + 256, ...; rows past the last pixel and
    // channels past C are written as zeros.  A neighbour outside the image
    // reads through an out-of-range buffer offset, which returns zeros.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)F.x_bytes, 0x00020000);
    const uint32_t colB = (uint32_t)C * 2u, rowB = (uint32_t)W * colB;
    int p = tid / F.c8, cg = tid - p * F.c8;
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
    // w+4, ...; the A operand is 16 weight rows, the B operand 16 pixels of d.
    // Lane l then holds outputs j0..j0+3 (j0 = 16*cb + 4*(l/16)) of pixel
    // 16*rb + l%16.
    const int kg = 8 * (lane >> 4);
    const bool quad = (NMASK & 3) == 0;   // 4 consecutive outputs of a pixel are 8-byte aligned in LDS
    for (int cb = wave; cb < F.ncb; cb += 4) {
        const T* wrow = omw + (long)min(cb * 16 + (lane & 15), F.NO - 1) * C;   // rows past NO compute a copy, not stored
        f4_t acc[MB];
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) acc[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int kk = 0; kk < F.KP; kk += 32) {
            const int k0 = kk + kg;
            const uint4 a = k0 < C ? *reinterpret_cast<const uint4*>(wrow + k0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) {
                const uint4 b = *reinterpret_cast<const uint4*>(A + (rb * 16 + (lane & 15)) * F.AST + k0);
                acc[rb] = mfma32<DT>(a, b, acc[rb]);
            }
        }
        const int j0 = cb * 16 + 4 * (lane >> 4);
        float bias[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[i] = to_f32(omb[min(j0 + i, F.NO - 1)]);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            const int row = rb * 16 + (lane & 15);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[rb][i] + bias[i];
            if (quad && j0 + 3 < NOFF) {
                *reinterpret_cast<uint2*>(Ooff + row * NOFF + j0) = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
            } else if (quad && j0 >= NOFF && j0 + 3 < F.NO) {
                *reinterpret_cast<uint2*>(Omask + row * NMASK + (j0 - NOFF)) =
                    make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = j0 + i;
                    if (j < NOFF) Ooff[row * NOFF + j] = from_f32<DT>(v[i]);
                    else if (j < F.NO) Omask[row * NMASK + (j - NOFF)] = from_f32<DT>(v[i]);
                }
            }
        }
    }
    __syncthreads();

    // ---- the tile's outputs are contiguous in both tensors
    copy_out(lds + F.o_off, reinterpret_cast<unsigned char*>(off + (long)px0 * NOFF), npx * NOFF * 2, tid);
    copy_out(lds + F.o_mask, reinterpret_cast<unsigned char*>(mask + (long)px0 * NMASK), npx * NMASK * 2, tid);
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

// Tile plan: the largest tile whose LDS keeps two workgroups per CU and that
// still gives two tiles per CU; else the largest that fits at all.  False if
// not even a 16-pixel tile fits.
bool plan_frontend(const Geom& G, int dtype, int lds_limit, int num_cus, FrontCfg* F)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    if (G.c % 8 != 0) return false;
    if ((long)G.n * G.h * G.w * G.c * 2 >= (1l << 31)) return false;   // buffer offsets, out-of-range marker 2^31
    for (int mb = 4; mb >= 1; mb /= 2) {
        layout(G, mb, F);
        if (F->lds_bytes <= std::min(FT_LDS_TARGET, lds_limit) && F->ntiles >= 2 * num_cus) return true;
    }
    for (int mb = 4; mb >= 1; mb /= 2) {
        layout(G, mb, F);
        if (F->lds_bytes <= lds_limit) return true;
    }
    return false;
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
    FrontCfg F;
    if (!plan_frontend(G, dtype, lds_limit, num_cus, &F)) return hipErrorInvalidValue;
    return dtype == DT_F16 ? launch_typed<DT_F16>(G, F, x, dww, dwb, omw, omb, off, mask, s)
                           : launch_typed<DT_BF16>(G, F, x, dww, dwb, omw, omb, off, mask, s);
}

}  // namespace dcn
