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
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo, hi;
            if constexpr (DT == DT_F16) {
                lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            } else {
                lo = from_f32<DT_BF16>(v[2 * i]);
                hi = from_f32<DT_BF16>(v[2 * i + 1]);
            }
            w[i] = lo | (hi << 16);
        }
        r.x = w[0]; r.y = w[1]; r.z = w[2]; r.w = w[3];
    }
    *reinterpret_cast<u32x4*>(p) = r;
}

// exp(z) for z <= 0 through the hardware base-2 exponential.
__device__ __forceinline__ float exp_nonpos(float z) { return exp2f(z * 1.44269504088896341f); }

// Scaled offsets whose magnitude reaches 2^24 (or that are not finite) put
// the sample outside any map this library accepts (h, w < 2^24).
__device__ __forceinline__ bool coord_ok(float t) { return fabsf(t) < 16777216.0f; }

}  // namespace dcn
