/*
 * dcn.h -- C ABI of libdcn: deformable sampling-and-aggregation on AMD
 * Instinct MI355X (gfx950).
 *
 * Operations, cited by web-page title and section:
 *
 *  dcn_forward   The DCN core operator.  For every output pixel p0 and channel
 *                group g:  y_g(p0) = sum_k m_gk * x_g(p0 + p_k + dp_gk)
 *                ("DCNv4: Unbounded Weights", "Why Is Sampling Just 9 Points
 *                Still Slow?").  x is read at the fractional point by bilinear
 *                interpolation with zero outside the map ("InternImage:
 *                Deformable Convolutions at Scale", Ch.2).  The modulation m
 *                is softmax-normalised over the K taps (DCNv3, same page Ch.3)
 *                or used as given (DCNv4, "DCNv4: Unbounded Weights",
 *                "1. Remove Softmax").  Groups: the C channels split into
 *                `group` groups of D = C/group channels sharing one set of K
 *                offsets and K modulations ("InternImage...", Ch.4).
 *  dcn_backward  Gradients of dcn_forward with respect to x, the offsets and
 *                the mask (the bilinear read is differentiable almost
 *                everywhere: "InternImage...", Ch.2, "Why bilinear, and why it
 *                is differentiable").
 *  msda_forward  Multi-scale deformable attention sampling core ("Deformable
 *                DETR: Learn Where to Read", "A learned location can fall
 *                between cells" and "Mix samples with a per-head budget"):
 *                per query and head, a softmax over all levels and points
 *                jointly, a bilinear read of every level at x = u*W_l - 1/2,
 *                y = v*H_l - 1/2 (zero outside, no clamping), and the
 *                weighted sum.
 *  msda_backward Gradients of msda_forward with respect to value, loc and
 *                attn (the read is differentiable in the location: "Deformable
 *                DETR...", "A learned location can fall between cells"; the
 *                joint softmax backward: "Mix samples with a per-head budget").
 *
 * Conventions (the pages leave these open; oracle and kernels hold them alike):
 *  - Tap k of a kernel_h x kernel_w grid sits at kx = k / kernel_h,
 *    ky = k % kernel_h (the grid is listed with the y component fastest).
 *  - Sampling point of tap k at output (ho, wo):
 *      px = wo*stride_w - pad_w + kx*dil_w + offset_scale*dx
 *      py = ho*stride_h - pad_h + ky*dil_h + offset_scale*dy
 *    Output size: ho = (h + 2*pad_h - (dil_h*(kernel_h-1)+1)) / stride_h + 1,
 *    likewise wo.
 *  - Accumulation is fp32; an f16/bf16 output is rounded once, to nearest even.
 *
 * Layouts (all dense, row-major, no strides):
 *    x        [n][h][w][c]                       (NHWC)
 *    offset   [n][ho][wo][group][K][2]           (dx, dy) in pixels, K = kernel_h*kernel_w
 *    mask     [n][ho][wo][group][K]              logits (softmax=1) or modulation (softmax=0)
 *    out      [n][ho][wo][c]
 *    value    [n][S][heads][head_dim]            levels flattened level-major, row-major
 *                                                within a level; S = sum_l H_l*W_l
 *    loc      [n][len_q][heads][levels][points][2]   normalised (u, v), u along the width
 *    attn     [n][len_q][heads][levels][points]      logits (softmax=1) or weights (softmax=0)
 *    msda out [n][len_q][heads][head_dim]
 *
 * Ownership and streams: every tensor pointer is a DEVICE pointer owned by the
 * caller (except msda_forward's spatial_shapes, a HOST array).  The library
 * allocates and frees nothing; its one device buffer of its own is the static
 * scratch array of dcn_backward_noalloc.  `stream` is a hipStream_t (NULL: the null
 * stream); every call only enqueues work on it and returns, and results are
 * ready when the stream is.  Calls are thread-safe.
 *
 * Errors: no exception crosses the ABI.  Invalid arguments return
 * DCN_ERR_INVALID before anything is enqueued, leaving outputs untouched;
 * dcn_last_error() then describes the problem (per thread).
 */
#ifndef LIBDCN_DCN_H
#define LIBDCN_DCN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DCN_OK = 0,
    DCN_ERR_INVALID = 1,      /* bad argument: NULL, size, shape, flag, dtype, overflow */
    DCN_ERR_UNSUPPORTED = 2,  /* well-formed but not provided (dtype of an op, alignment, levels) */
    DCN_ERR_HIP = 3           /* the HIP runtime reported an error at launch */
} dcn_status;

typedef enum { DCN_F32 = 0, DCN_F16 = 1, DCN_BF16 = 2 } dcn_dtype;

typedef struct {
    int32_t n, h, w, c, group;          /* x is [n][h][w][c]; c % group == 0 */
    int32_t kernel_h, kernel_w;         /* >= 1 */
    int32_t stride_h, stride_w;         /* >= 1 */
    int32_t pad_h, pad_w;               /* >= 0 */
    int32_t dil_h, dil_w;               /* >= 1 */
    float offset_scale;                 /* multiplies every offset before it is added; finite */
    int32_t softmax;                    /* 1: DCNv3 (softmax over K); 0: DCNv4 (as given) */
    int32_t dtype;                      /* dcn_dtype of x, offset, mask, out and all grads */
} dcn_desc;

typedef struct {
    int32_t n, len_q, heads, head_dim, levels, points;   /* all >= 1; levels <= 16 */
    int32_t softmax;                                     /* 1: attn holds logits */
    int32_t dtype;                                       /* DCN_F32 only */
} msda_desc;

/* Output size of dcn_forward for `desc` (ordinary convolution geometry).
 * Returns DCN_ERR_INVALID if the geometry is invalid or either size < 1. */
dcn_status dcn_output_size(const dcn_desc* desc, int32_t* h_out, int32_t* w_out);

/* out = DCN core op (see above).  x, offset, mask, out: device pointers,
 * aligned to the element size, in desc->dtype (f32, f16 or bf16).
 * Every element count must be below 2^31 and h, w below 2^24.  An offset
 * whose scaled magnitude reaches 2^24, or that is not finite, places its
 * sample outside the map (it contributes zero). */
dcn_status dcn_forward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                       void* out, void* stream);

/* Gradients of dcn_forward given grad_out ([n][ho][wo][c]).  All tensors are
 * in desc->dtype (f32, f16 or bf16); arithmetic is fp32.  grad_x
 * ([n][h][w][c]) is OVERWRITTEN: its fp32 sums are zero-filled on `stream`,
 * then accumulated partly with fp32 atomics, so their low bits depend on the
 * order of the atomics.  grad_offset and grad_mask (same layouts as offset and
 * mask) are overwritten; with softmax=1 grad_mask is the gradient with respect
 * to the logits passed in `mask`.  f16/bf16 results are rounded once, to
 * nearest even.  Any of grad_x, grad_offset, grad_mask may be NULL to skip
 * it.  At a sample coordinate that is exactly an integer the derivative of the
 * cell above the floor (the right-hand derivative) is returned.
 * An f16/bf16 backward that computes grad_x sums it in an fp32 buffer the
 * caller provides: use dcn_backward_ws.  dcn_backward is dcn_backward_ws with
 * no workspace, so for f16/bf16 with grad_x it returns DCN_ERR_INVALID. */
dcn_status dcn_backward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                        const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask,
                        void* stream);

/* Bytes of device workspace dcn_backward_ws needs for `desc` when grad_x is
 * computed: 4*n*h*w*c for f16/bf16 (the fp32 sums of grad_x), 0 for f32.
 * Half-precision backward is the DCNv4 training case ("DCNv4: Unbounded
 * Weights", "2. Move Less Data on the GPU": half precision halves the bytes
 * moved). */
dcn_status dcn_backward_workspace_size(const dcn_desc* desc, size_t* bytes);

/* dcn_backward with a caller-owned device workspace (4-byte aligned, at least
 * dcn_backward_workspace_size bytes; may be NULL when that size is 0 or
 * grad_x is NULL).  Its contents on entry do not matter and are clobbered;
 * calls that share a workspace must not overlap in time. */
dcn_status dcn_backward_ws(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                           const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask,
                           void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * dcn_backward_ws with no workspace argument.  The fp32 sums of an f16/bf16
 * grad_x live in a device array the library owns, 64 MiB per GPU (held from
 * the first call on that GPU until the process ends), so grad_x may have at
 * most 16 Mi elements (n*h*w*c <= 16777216); a larger f16/bf16 grad_x is
 * DCN_ERR_INVALID before anything is enqueued.  f32, or grad_x NULL, uses no
 * scratch.  The call allocates nothing: it enqueues the same kernels as
 * dcn_backward_ws (the scratch is zero-filled by a kernel on `stream`, not
 * by a memset).  Its first call on a device looks up the array's address
 * (hipGetSymbolAddress, which may load the library's code object): make that
 * first call outside any graph capture.  Every call on one GPU shares that
 * GPU's array, so calls that overlap in time on one GPU (different streams,
 * or threads) race and must be serialised by the caller.  Everything else,
 * arguments and results included, is as dcn_backward_ws. */
dcn_status dcn_backward_noalloc(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask,
                                void* stream);

/* DCNv4 front-end: the offsets and modulation of the core op computed from
 * the module input x ("DCNv4: Unbounded Weights", "1. Remove Softmax": the
 * offset and weight linears merge into one, and the offset subnetwork is a
 * depthwise 3x3 convolution followed by that linear, with no LayerNorm or
 * GELU between).  For every pixel of x ([n][h][w][c]):
 *   d  = depthwise 3x3 of x, stride 1, zero padding 1:
 *        d[c] = dw_bias[c] + sum_{i,j} dw_weight[i][j][c] * x[y+i-1][x+j-1][c]
 *   om = om_weight d + om_bias         (om_weight [group*K*3][c], a linear layer's
 *                                       [out][in] layout; om_bias [group*K*3])
 *   offset[g][k][a] = om[(g*K + k)*2 + a],  mask[g][k] = om[group*K*2 + g*K + k]
 * with K = kernel_h*kernel_w; offset and mask take the layouts dcn_forward
 * reads.  d is rounded to desc->dtype before the linear layer (on the matrix
 * cores, fp32 sums); each output is rounded once.  desc->dtype must be f16 or
 * bf16, c % 8 == 0, and the core's output must have the input's size
 * (stride 1, (kernel-1)*dil == 2*pad); otherwise DCN_ERR_UNSUPPORTED, as when
 * c and group*K*3 exceed the kernel's LDS tiles.  x, dw_weight, dw_bias,
 * om_weight, offset and mask must be 16-byte aligned. */
dcn_status dcn_offset_mask(const dcn_desc* desc, const void* x, const void* dw_weight, const void* dw_bias,
                           const void* om_weight, const void* om_bias, void* offset, void* mask, void* stream);

/* Multi-scale deformable attention sampling core (see above).
 * spatial_shapes: HOST array [levels][2] = (H_l, W_l), each >= 1.
 * value, loc, attn, out: device pointers in f32.  Element counts below 2^31. */
dcn_status msda_forward(const msda_desc* desc, const int32_t* spatial_shapes, const void* value,
                        const void* loc, const void* attn, void* out, void* stream);

/* msda_forward with the sampling locations formed in the kernel from
 * references, valid ratios and offsets, and with padded value cells ("Deformable
 * DETR: Learn Where to Read", "A reference links resolutions without equating
 * their pixels", "A learned location can fall between cells" on box
 * references, and "Math and tensor shapes"):
 *   reference    [n][len_q][ref_dims], f32, in valid-image normalised
 *                coordinates: (x, y) for ref_dims 2, (x, y, w, h) for 4;
 *   valid_ratios [n][levels][2] = (valid W / W_l, valid H / H_l), f32, or NULL
 *                for ratios of 1;
 *   offsets      [n][len_q][heads][levels][points][2], f32 (the loc layout);
 *   padding_mask [n][S] bytes, nonzero = padded value cell, or NULL.
 * Sample (l, p) of a query with level ratios (r_w, r_h) is read at
 *   ref_dims 2:  u = x r_w + dx / W_l,              v = y r_h + dy / H_l
 *   ref_dims 4:  u = x r_w + (dx / points) w r_w / 2, v = y r_h + (dy / points) h r_h / 2
 * (formed in fp64), then exactly as msda_forward reads loc = (u, v), except
 * that a padded cell reads zero (the attention module zeroes projected values
 * at masked positions).  attn, out and the other requirements are those of
 * msda_forward; ref_dims other than 2 or 4 is DCN_ERR_INVALID. */
dcn_status msda_forward_ref(const msda_desc* desc, const int32_t* spatial_shapes, int32_t ref_dims,
                            const void* value, const void* reference, const void* valid_ratios,
                            const void* offsets, const void* attn, const uint8_t* padding_mask, void* out,
                            void* stream);

/* Gradients of msda_forward given grad_out ([n][len_q][heads][head_dim]).
 * grad_value ([n][S][heads][head_dim]) is OVERWRITTEN: zero-filled on
 * `stream`, then accumulated with fp32 atomics, so its low bits depend on the
 * order of the atomics.  grad_loc and grad_attn (the layouts of loc and attn)
 * are overwritten; with softmax=1 grad_attn is the gradient with respect to
 * the logits passed in `attn`.  Any of grad_value, grad_loc, grad_attn may be
 * NULL to skip it.  A sample that falls outside its level has zero location
 * gradient; at a coordinate that is exactly an integer the derivative of the
 * cell above the floor (the right-hand derivative) is returned.
 * desc->dtype must be DCN_F32 (otherwise DCN_ERR_UNSUPPORTED); the other
 * requirements are those of msda_forward. */
dcn_status msda_backward(const msda_desc* desc, const int32_t* spatial_shapes, const void* value,
                         const void* loc, const void* attn, const void* grad_out, void* grad_value,
                         void* grad_loc, void* grad_attn, void* stream);

/* Bytes of device workspace msda_backward_ws needs for grad_value to be
 * gathered per value cell rather than scattered with atomics (same gradients;
 * "Deformable DETR: Learn Where to Read", "A learned location can fall between
 * cells": a cell's value gradient is the sum, over the samples it is a corner
 * of, of the corner weight times the attention weight times grad_out).  0
 * when the shape has no gather path (head_dim not a power of two in 4..64,
 * levels*points not a power of two up to 32, grad_out of 2 GiB or more) or
 * desc->dtype is not f32.  At the Deformable DETR encoder shape (n=8,
 * S=len_q=17821, 8 heads, 4 levels x 4 points) it is about 370 MB: 20 bytes
 * per sample plus 4 bytes per cell of a (H_l+1) x (W_l+1) grid per level,
 * image and head. */
dcn_status msda_backward_workspace_size(const msda_desc* desc, const int32_t* spatial_shapes, size_t* bytes);

/* msda_backward with a caller-owned device workspace (256-byte aligned, at
 * least msda_backward_workspace_size bytes when grad_value is requested and
 * that size is nonzero; otherwise it may be NULL and is not used).  With a
 * workspace, grad_value is written once per cell, without atomics and without
 * a zero-fill; the order in which a cell's contributions are summed still
 * depends on the order of the counting atomics, so its low bits may differ
 * from run to run.  A missing or short workspace is DCN_ERR_INVALID, a
 * misaligned one DCN_ERR_UNSUPPORTED.  grad_value or grad_out that is not
 * 16-byte aligned (or a loc / grad_loc that is not 8-byte aligned) takes the
 * atomic scatter instead.  Calls that share a workspace must not overlap in
 * time.  Everything else is as msda_backward. */
dcn_status msda_backward_ws(const msda_desc* desc, const int32_t* spatial_shapes, const void* value,
                            const void* loc, const void* attn, const void* grad_out, void* grad_value,
                            void* grad_loc, void* grad_attn, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static name of a status code. */
const char* dcn_status_str(dcn_status status);

/* Description of the last error returned on the calling thread ("" if none). */
const char* dcn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBDCN_DCN_H */
