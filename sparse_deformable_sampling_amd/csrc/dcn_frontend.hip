// DCNv4 front-end for gfx950: the offsets and modulation the core op reads,
// produced from the module input x.
//
// "DCNv4: Unbounded Weights", "1. Remove Softmax": with the softmax gone the
// offsets and the modulation come from ONE linear layer, and the offset
// subnetwork is a separable convolution: a depthwise 3x3 convolution, then
// that linear layer (no LayerNorm or GELU between them).  So for every pixel
//   d   = depthwise3x3(x)                       (stride 1, zero padding 1)
//   om  = d . W_om + b_om                       (C -> G*K*3 outputs)
//   offset[g][k][0..1] = om[(g*K + k)*2 + 0..1],  mask[g][k] = om[G*K*2 + g*K + k].
//
// Work split: persistent workgroups of four waves walk over tiles of 64
// pixels of one image row.
//  - The depthwise convolution of a tile: a thread takes (pixel, 8
//    channels), reads the 3x3 neighbourhood with 16-byte loads (cache hits
//    for the overlapping rows), sums in fp32 and writes d, rounded once to
//    the storage type, into an LDS tile A[64][C] (rows padded by 16 bytes so
//    that the MFMA operand reads of 16 rows spread over the banks).
//  - The linear layer is a 64 x C by C x (G*K*3) product on the matrix
//    cores: v_mfma_f32_16x16x16 (f16 or bf16 inputs, fp32 sums).  W_om is
//    staged transposed in LDS (Bt[out][C]), 128 output columns at a time; with
//    one such chunk it is loaded once per workgroup and kept.
//  - Epilogue: the bias is added in fp32 and each value is rounded once into
//    the offset or mask tensor.
#include <algorithm>

#include "dcn_device.h"
#include "dcn_launch.h"
#include "dcn_ring.h"

namespace dcn {

namespace {

constexpr int FT_M = 64;     // pixels per tile
constexpr int FT_NB = 128;   // output columns per staged weight chunk

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

struct FrontCfg {
    int KP;        // C rounded up to 16 (the MFMA k extent)
    int AST;       // A tile row stride in elements (KP + 8)
    int NO;        // G*K*3 outputs
    int NOP;       // NO rounded up to 16
    int NB;        // output columns per chunk (<= FT_NB, a multiple of 16)
    int nchunks;   // chunks of NB columns
    int tiles_w;   // tiles per image row
    int ntiles;    // n * h * tiles_w
    int nwg;
    int lds_bytes;
};

// One 16x16x16 product-accumulate with operands held as 4 storage-type values.
template <int DT>
__device__ __forceinline__ f4_t mfma16(uint2 a, uint2 b, f4_t c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a), __builtin_bit_cast(h4_t, b), c, 0, 0,
                                                     0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b), c,
                                                         0, 0, 0);
}

template <int DT>
__global__ __launch_bounds__(256) void dcn_offset_mask_k(Geom G, FrontCfg F, const typename Elem<DT>::T* __restrict__ x,
                                                         const typename Elem<DT>::T* __restrict__ dww,
                                                         const typename Elem<DT>::T* __restrict__ dwb,
                                                         const typename Elem<DT>::T* __restrict__ omw,
                                                         const typename Elem<DT>::T* __restrict__ omb,
                                                         typename Elem<DT>::T* __restrict__ off,
                                                         typename Elem<DT>::T* __restrict__ mask)
{
    using T = typename Elem<DT>::T;
    extern __shared__ __align__(16) unsigned char lds[];
    T* A = reinterpret_cast<T*>(lds);                                  // [FT_M][AST]
    T* Bt = reinterpret_cast<T*>(lds + (size_t)FT_M * F.AST * sizeof(T));   // [NB][AST]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = G.c, H = G.h, W = G.w;
    const int NOFF = G.g * G.K * 2;     // offset outputs per pixel
    const int c8 = F.KP / 8;            // 8-channel groups of a row of A (incl. the zero pad)

    // Weight chunk q (output columns q*NB ...) into Bt, zero beyond NO and C.
    auto load_b = [&](int q) {
        for (int e = tid; e < F.NB * F.KP; e += 256) {
            const int jl = e / F.KP, k = e - jl * F.KP;
            const int j = q * F.NB + jl;
            Bt[jl * F.AST + k] = (j < F.NO && k < C) ? omw[(long)k * F.NO + j] : from_f32<DT>(0.f);
        }
    };
    if (F.nchunks == 1) load_b(0);

    for (int t = blockIdx.x; t < F.ntiles; t += gridDim.x) {
        const int tw = t % F.tiles_w, ny = t / F.tiles_w;
        const int y = ny % H, n = ny / H;
        const int px0 = tw * FT_M;
        // ---- depthwise 3x3 into A
        for (int e = tid; e < FT_M * c8; e += 256) {
            const int p = e / c8, cc = (e - p * c8) * 8;
            const int xc = px0 + p;
            float acc[8];
            if (xc < W && cc < C) {
                load_vec<DT>(dwb + cc, acc);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int yy = y + i - 1;
                    if ((unsigned)yy >= (unsigned)H) continue;
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        const int xx = xc + j - 1;
                        if ((unsigned)xx >= (unsigned)W) continue;
                        float xv[8], wv[8];
                        load_vec<DT>(x + (((long)n * H + yy) * W + xx) * C + cc, xv);
                        load_vec<DT>(dww + (long)(i * 3 + j) * C + cc, wv);
#pragma unroll
                        for (int u = 0; u < 8; ++u) acc[u] = fmaf(wv[u], xv[u], acc[u]);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) acc[u] = 0.f;
            }
            store_vec<DT>(A + p * F.AST + cc, acc);
        }
        for (int q = 0; q < F.nchunks; ++q) {
            if (F.nchunks > 1) load_b(q);
            __syncthreads();
            // ---- 64 x NB block of the product: wave w takes column blocks w, w+4, ...
            const int nbl = F.NB / 16;
            for (int nb = wave; nb < nbl; nb += 4) {
                f4_t c[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) c[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
                const T* bp = Bt + (nb * 16 + (lane & 15)) * F.AST + 4 * (lane >> 4);
                for (int kk = 0; kk < F.KP; kk += 16) {
                    const uint2 b = *reinterpret_cast<const uint2*>(bp + kk);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) {
                        const uint2 a =
                            *reinterpret_cast<const uint2*>(A + (mb * 16 + (lane & 15)) * F.AST + 4 * (lane >> 4) + kk);
                        c[mb] = mfma16<DT>(a, b, c[mb]);
                    }
                }
                // ---- epilogue: row 4*(lane/16)+i of block mb is pixel mb*16 + that row; column lane%16
                const int j = q * F.NB + nb * 16 + (lane & 15);
                if (j < F.NO) {
                    const float bias = to_f32(omb[j]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int xc = px0 + mb * 16 + 4 * (lane >> 4) + i;
                            if (xc >= W) continue;
                            const long pix = ((long)n * H + y) * W + xc;
                            const T v = from_f32<DT>(c[mb][i] + bias);
                            if (j < NOFF) off[pix * NOFF + j] = v;
                            else mask[pix * (NOFF / 2) + (j - NOFF)] = v;
                        }
                }
            }
            __syncthreads();   // A (next tile) and Bt (next chunk) are rewritten next
        }
    }
}

template <int DT>
hipError_t launch_typed(const Geom& G, const FrontCfg& F, const void* x, const void* dww, const void* dwb,
                        const void* omw, const void* omb, void* off, void* mask, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    auto* fn = dcn_offset_mask_k<DT>;
    const hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, F.lds_bytes);
    if (e != hipSuccess) return e;
    fn<<<dim3(F.nwg), dim3(256), F.lds_bytes, s>>>(G, F, (const T*)x, (const T*)dww, (const T*)dwb, (const T*)omw,
                                                   (const T*)omb, (T*)off, (T*)mask);
    return hipGetLastError();
}

}  // namespace

namespace {

// Tile plan; false if even a 16-column weight chunk does not fit in LDS.
bool plan_frontend(const Geom& G, int dtype, int lds_limit, int num_cus, FrontCfg* F)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    if (G.c % 8 != 0) return false;
    F->KP = (G.c + 15) / 16 * 16;
    F->AST = F->KP + 8;
    F->NO = G.g * G.K * 3;
    F->NOP = (F->NO + 15) / 16 * 16;
    // widest chunk (a multiple of 16, at most FT_NB) whose tiles fit
    F->NB = std::min(F->NOP, FT_NB);
    while (F->NB > 16 && (long)(FT_M + F->NB) * F->AST * 2 > lds_limit) F->NB -= 16;
    F->lds_bytes = (FT_M + F->NB) * F->AST * 2;
    if (F->lds_bytes > lds_limit) return false;
    F->nchunks = (F->NOP + F->NB - 1) / F->NB;
    F->tiles_w = (G.w + FT_M - 1) / FT_M;
    F->ntiles = G.n * G.h * F->tiles_w;
    F->nwg = std::min(F->ntiles, num_cus * 2);
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
    FrontCfg F;
    if (!plan_frontend(G, dtype, lds_limit, num_cus, &F)) return hipErrorInvalidValue;
    if (F.ntiles == 0) return hipSuccess;
    return dtype == DT_F16 ? launch_typed<DT_F16>(G, F, x, dww, dwb, omw, omb, off, mask, s)
                           : launch_typed<DT_BF16>(G, F, x, dww, dwb, omw, omb, off, mask, s);
}

}  // namespace dcn
