// Internal interface between the C-ABI layer (dcn_api.hip) and the kernel
// launchers.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcn {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Validated DCN geometry, passed to kernels by value.
struct Geom {
    int n, h, w, c, g, d;           // d = c / g
    int kh, kw, sh, sw, ph, pw, dh, dw;
    int ho, wo, K;                  // K = kh * kw
    int items;                      // n * ho * wo * g  (one item = one (pixel, group))
    float scale;                    // offset_scale
    int softmax;
};

constexpr int MSDA_MAX_LEVELS = 16;

struct MsdaGeom {
    int n, q, m, dh, L, P;          // batch, queries, heads, head dim, levels, points
    int S;                          // sum of H_l * W_l
    int softmax;
    int H[MSDA_MAX_LEVELS], W[MSDA_MAX_LEVELS], start[MSDA_MAX_LEVELS];
    double inv_w[MSDA_MAX_LEVELS], inv_h[MSDA_MAX_LEVELS];   // 1 / W_l, 1 / H_l
    double half_inv_p;                                       // 0.5 / P
};

// Each returns hipSuccess or the launch error.
hipError_t launch_dcn_forward(const Geom& g, int dtype, const void* x, const void* off, const void* mask,
                              void* out, hipStream_t s);
// x, off, mask, gout, gx, goff, gmask in the storage type dtype.  grad_x is
// summed in fp32: in gx itself for f32, else in ws (n*h*w*c floats, needed
// only when gx is requested), which is then rounded into gx.
hipError_t launch_dcn_backward(const Geom& g, int dtype, const void* x, const void* off, const void* mask,
                               const void* gout, void* gx, void* goff, void* gmask, float* ws, hipStream_t s);
// DCNv4 front-end (dcn_frontend.hip): depthwise 3x3 of x, then the merged
// offset+mask linear, into the core's offset and mask layouts.  f16/bf16,
// c % 8 == 0; frontend_supported tells whether the LDS tiles fit.
bool frontend_supported(const Geom& g, int dtype, int lds_limit);
hipError_t launch_dcn_offset_mask(const Geom& g, int dtype, const void* x, const void* dww, const void* dwb,
                                  const void* omw, const void* omb, void* off, void* mask, hipStream_t s);
hipError_t launch_msda_forward(const MsdaGeom& g, const float* value, const float* loc, const float* attn,
                               float* out, hipStream_t s);
// Locations formed in the kernel from a point (ref_dims 2) or box (4)
// reference per query, valid ratios [n][L][2] (or NULL: 1) and offsets laid
// out like loc; pad [n][S] (or NULL) marks value cells that read zero.
hipError_t launch_msda_forward_ref(const MsdaGeom& g, int ref_dims, const float* value, const float* ref,
                                   const float* ratios, const float* offsets, const float* attn,
                                   const uint8_t* pad, float* out, hipStream_t s);
// With a workspace of at least msda_backward_workspace(g) bytes (0: the shape
// has no gather path), grad_value is gathered per cell; otherwise it is
// zero-filled and scattered with atomics.
size_t msda_backward_workspace(const MsdaGeom& g);
hipError_t launch_msda_backward(const MsdaGeom& g, const float* value, const float* loc, const float* attn,
                                const float* gout, float* gvalue, float* gloc, float* gattn, void* ws,
                                size_t ws_bytes, hipStream_t s);

#ifdef DCN_COUNT_WRITES
// Debug build only (libdcn_count.so): point the output-write counter of the
// forward kernels' translation units at counts[0..n] for the output buffer
// `base` of n elements of es bytes (counts == NULL: stop counting).
hipError_t ring_count_writes(unsigned int* counts, const void* base, unsigned long long n, unsigned int es);
hipError_t fwd_count_writes(unsigned int* counts, const void* base, unsigned long long n, unsigned int es);
hipError_t msda_count_writes(unsigned int* counts, const void* base, unsigned long long n, unsigned int es);
hipError_t frontend_count_writes(unsigned int* counts, const void* base, unsigned long long n, unsigned int es);
#endif

}  // namespace dcn
