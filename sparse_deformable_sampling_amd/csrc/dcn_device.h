// Device-side helpers shared by the libdcn kernels (internal header).
//
// Storage types: f32, f16 (_Float16) and bf16 (kept as its uint16 bit
// pattern).  All arithmetic is fp32; an f16/bf16 result is rounded once, to
// nearest even, when it is stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_launch.h"

namespace dcn {

#ifdef DCN_COUNT_WRITES
// Debug build only: every store of an op output also adds one, per element
// written, to counts[i] for element i of the registered output buffer, or to
// counts[n] for an address outside it, so the host can check that each
// output element of an atomic-free kernel has exactly one writer and that no
// store lands elsewhere.  Each translation unit holds its own registration
// (NULL counts: nothing is counted, as in translation units that never
// register one).  Stores to LDS are never counted.
struct WriteCounts {
    unsigned int* counts;
    unsigned long long base, n;
    unsigned int es;
};
static __device__ WriteCounts g_write_counts;

__device__ __forceinline__ void count_writes(const void* p, int elems)
{
    const WriteCounts w = g_write_counts;
    if (!w.counts || __builtin_amdgcn_is_shared((const __attribute__((address_space(0))) void*)p)) return;   // LDS stores are not outputs
    for (int i = 0; i < elems; ++i) {
        const unsigned long long a = (unsigned long long)p + (unsigned long long)i * w.es;
        const bool in = a >= w.base && (a - w.base) % w.es == 0 && (a - w.base) / w.es < w.n;
        atomicAdd(w.counts + (in ? (a - w.base) / w.es : w.n), 1u);
    }
}

#define DCN_WRITE_COUNT_SETTER(name)                                                                        \
    hipError_t name(unsigned int* counts, const void* base, unsigned long long n, unsigned int es)          \
    {                                                                                                       \
        const WriteCounts w = {counts, (unsigned long long)base, n, es};                                   \
        return hipMemcpyToSymbol(HIP_SYMBOL(g_write_counts), &w, sizeof w);                                 \
    }
#else
__device__ __forceinline__ void count_writes(const void*, int) {}
#endif

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; };
template <> struct Elem<DT_F16> { using T = _Float16; };
template <> struct Elem<DT_BF16> { using T = uint16_t; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <int DT> __device__ __forceinline__ typename Elem<DT>::T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<DT_F32>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<DT_F16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ uint16_t from_f32<DT_BF16>(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 values rounded to nearest even into one dword of the 16-bit
// storage type, the first in the low half: gfx950's packed conversions (one
// instruction for the pair; the f16 one rounds exactly as v_cvt_f16_f32, the
// bf16 one as the bit-level rounding of from_f32<DT_BF16>).
template <int DT>
__device__ __forceinline__ uint32_t pack2_rne(float lo, float hi)
{
    uint32_t r;
    if constexpr (DT == DT_F16)
        asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    else
        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// Channels per 16-byte vector.
template <int DT> struct Vec { static constexpr int N = 16 / (int)sizeof(typename Elem<DT>::T); };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load one 16-byte vector (V = 16/sizeof(T) channels) and widen it to fp32.
template <int DT>
__device__ __forceinline__ void load_vec(const typename Elem<DT>::T* p, float* v)
{
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
    if constexpr (DT == DT_F32) {
        v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
    } else if constexpr (DT == DT_F16) {
        uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    } else {
        uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// Round fp32 values to the storage type and write one 16-byte vector.
template <int DT>
__device__ __forceinline__ void store_vec(typename Elem<DT>::T* p, const float* v)
{
    u32x4 r;
    if constexpr (DT == DT_F32) {
        r.x = __float_as_uint(v[0]); r.y = __float_as_uint(v[1]);
        r.z = __float_as_uint(v[2]); r.w = __float_as_uint(v[3]);
    } else {
        r.x = pack2_rne<DT>(v[0], v[1]);
        r.y = pack2_rne<DT>(v[2], v[3]);
        r.z = pack2_rne<DT>(v[4], v[5]);
        r.w = pack2_rne<DT>(v[6], v[7]);
    }
    *reinterpret_cast<u32x4*>(p) = r;
    count_writes(p, 16 / (int)sizeof(typename Elem<DT>::T));
}

// Max or sum over aligned groups of w lanes (w a power of two, every lane of
// a group active), each lane of a group ending with the group's result: DPP
// moves within a row of 16 (neighbours, pairs, then mirrors within 8 and 16
// lanes), which stay in the VALU, and cross-lane shuffles beyond 16.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float group_reduce(float v, int w)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if (w >= 2) v = op(v, dpp_read<0xB1>(v));    // quad_perm [1,0,3,2]
    if (w >= 4) v = op(v, dpp_read<0x4E>(v));    // quad_perm [2,3,0,1]
    if (w >= 8) v = op(v, dpp_read<0x141>(v));   // half-row mirror
    if (w >= 16) v = op(v, dpp_read<0x140>(v));  // row mirror
    for (int o = 16; o < w; o <<= 1) v = op(v, __shfl_xor(v, o, 64));
    return v;
}

// exp(z) for z <= 0 through the hardware base-2 exponential.
__device__ __forceinline__ float exp_nonpos(float z) { return exp2f(z * 1.44269504088896341f); }

// Scaled offsets whose magnitude reaches 2^24 (or that are not finite) put
// the sample outside any map this library accepts (h, w < 2^24).
__device__ __forceinline__ bool coord_ok(float t) { return fabsf(t) < 16777216.0f; }

}  // namespace dcn
