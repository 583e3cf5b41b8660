// C ABI of libdcn (declared in include/dcn.h): argument validation and
// dispatch to the kernel launchers.  Validation happens entirely on the host
// before anything is enqueued; on failure no output is touched.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/dcn.h"
#include "dcn_launch.h"
#include "dcn_ring.h"
#ifdef DCN_COUNT_WRITES
#include "../../include/dcn_debug.h"
#endif

namespace {

thread_local char g_last_error[512] = "";

dcn_status fail(dcn_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

dcn_status ok()
{
    g_last_error[0] = '\0';
    return DCN_OK;
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;   // element counts must stay below 2^31
constexpr int32_t kMaxSide = 1 << 24;             // h, w below 2^24

size_t elem_size(int32_t dt) { return dt == DCN_F32 ? 4 : 2; }

dcn_status check_ptr(const void* p, const char* name, size_t align)
{
    if (!p) return fail(DCN_ERR_INVALID, "%s is NULL", name);
    if ((uintptr_t)p % align) return fail(DCN_ERR_UNSUPPORTED, "%s is not aligned to %zu bytes", name, align);
    return DCN_OK;
}

// Validate a dcn_desc and fill the kernel geometry.
dcn_status make_geom(const dcn_desc* d, dcn::Geom* G)
{
    if (!d) return fail(DCN_ERR_INVALID, "desc is NULL");
    if (d->n < 1 || d->h < 1 || d->w < 1 || d->c < 1 || d->group < 1)
        return fail(DCN_ERR_INVALID, "n, h, w, c and group must be >= 1 (got %d, %d, %d, %d, %d)", d->n, d->h, d->w,
                    d->c, d->group);
    if (d->c % d->group)
        return fail(DCN_ERR_INVALID, "c (%d) is not a multiple of group (%d)", d->c, d->group);
    if (d->kernel_h < 1 || d->kernel_w < 1 || d->stride_h < 1 || d->stride_w < 1 || d->dil_h < 1 || d->dil_w < 1)
        return fail(DCN_ERR_INVALID, "kernel, stride and dilation must be >= 1");
    if (d->pad_h < 0 || d->pad_w < 0) return fail(DCN_ERR_INVALID, "padding must be >= 0");
    if (d->h >= kMaxSide || d->w >= kMaxSide) return fail(DCN_ERR_INVALID, "h and w must be below 2^24");
    if (d->softmax != 0 && d->softmax != 1) return fail(DCN_ERR_INVALID, "softmax must be 0 or 1");
    if (d->dtype != DCN_F32 && d->dtype != DCN_F16 && d->dtype != DCN_BF16)
        return fail(DCN_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (!isfinite(d->offset_scale)) return fail(DCN_ERR_INVALID, "offset_scale must be finite");
    const int64_t K = (int64_t)d->kernel_h * d->kernel_w;
    const int64_t eh = (int64_t)d->dil_h * (d->kernel_h - 1) + 1, ew = (int64_t)d->dil_w * (d->kernel_w - 1) + 1;
    const int64_t hp = (int64_t)d->h + 2 * (int64_t)d->pad_h, wp = (int64_t)d->w + 2 * (int64_t)d->pad_w;
    if (hp < eh || wp < ew) return fail(DCN_ERR_INVALID, "kernel extent exceeds the padded input");
    const int64_t ho = (hp - eh) / d->stride_h + 1, wo = (wp - ew) / d->stride_w + 1;
    if (ho < 1 || wo < 1 || ho >= kMaxSide || wo >= kMaxSide) return fail(DCN_ERR_INVALID, "invalid output size");
    const int64_t nx = (int64_t)d->n * d->h * d->w * d->c;
    const int64_t nout = (int64_t)d->n * ho * wo * d->c;
    const int64_t nmask = (int64_t)d->n * ho * wo * d->group * K;
    if (nx >= kMaxElems || nout >= kMaxElems || nmask * 2 >= kMaxElems || K >= kMaxElems)
        return fail(DCN_ERR_INVALID, "an element count reaches 2^31");
    G->n = d->n; G->h = d->h; G->w = d->w; G->c = d->c; G->g = d->group; G->d = d->c / d->group;
    G->kh = d->kernel_h; G->kw = d->kernel_w; G->sh = d->stride_h; G->sw = d->stride_w;
    G->ph = d->pad_h; G->pw = d->pad_w; G->dh = d->dil_h; G->dw = d->dil_w;
    G->ho = (int)ho; G->wo = (int)wo; G->K = (int)K;
    G->items = (int)((int64_t)d->n * ho * wo * d->group);
    G->scale = d->offset_scale;
    G->softmax = d->softmax;
    return DCN_OK;
}

dcn_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return ok();
    return fail(DCN_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* dcn_status_str(dcn_status s)
{
    switch (s) {
        case DCN_OK: return "DCN_OK";
        case DCN_ERR_INVALID: return "DCN_ERR_INVALID";
        case DCN_ERR_UNSUPPORTED: return "DCN_ERR_UNSUPPORTED";
        case DCN_ERR_HIP: return "DCN_ERR_HIP";
    }
    return "DCN_UNKNOWN_STATUS";
}

const char* dcn_last_error(void) { return g_last_error; }

dcn_status dcn_output_size(const dcn_desc* desc, int32_t* h_out, int32_t* w_out)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    if (!h_out || !w_out) return fail(DCN_ERR_INVALID, "h_out/w_out is NULL");
    *h_out = G.ho;
    *w_out = G.wo;
    return ok();
}

dcn_status dcn_forward(const dcn_desc* desc, const void* x, const void* offset, const void* mask, void* out,
                       void* stream)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    const size_t es = elem_size(desc->dtype);
    if ((st = check_ptr(x, "x", es)) || (st = check_ptr(offset, "offset", es)) ||
        (st = check_ptr(mask, "mask", es)) || (st = check_ptr(out, "out", es)))
        return st;
    return hip_status(dcn::launch_dcn_forward(G, desc->dtype, x, offset, mask, out, (hipStream_t)stream));
}

// Bytes of fp32 workspace a backward of this geometry and dtype needs for
// its grad_x sums (0 for f32, where grad_x itself holds them).
static int64_t backward_ws_bytes(const dcn_desc* d)
{
    return d->dtype == DCN_F32 ? 0 : (int64_t)d->n * d->h * d->w * d->c * 4;
}

// Pointer checks of a backward call (the geometry is already valid).
static dcn_status check_backward_ptrs(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                      const void* grad_out, const void* grad_x, const void* grad_offset,
                                      const void* grad_mask)
{
    dcn_status st;
    const size_t es = elem_size(desc->dtype);
    if ((st = check_ptr(x, "x", es)) || (st = check_ptr(offset, "offset", es)) ||
        (st = check_ptr(mask, "mask", es)) || (st = check_ptr(grad_out, "grad_out", es)))
        return st;
    if (grad_x && (uintptr_t)grad_x % es) return fail(DCN_ERR_UNSUPPORTED, "grad_x is not aligned");
    if (grad_offset && (uintptr_t)grad_offset % es) return fail(DCN_ERR_UNSUPPORTED, "grad_offset is not aligned");
    if (grad_mask && (uintptr_t)grad_mask % es) return fail(DCN_ERR_UNSUPPORTED, "grad_mask is not aligned");
    return DCN_OK;
}

static dcn_status backward_impl(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    if ((st = check_backward_ptrs(desc, x, offset, mask, grad_out, grad_x, grad_offset, grad_mask))) return st;
    const int64_t need = grad_x ? backward_ws_bytes(desc) : 0;
    if (need > 0) {
        if (!workspace)
            return fail(DCN_ERR_INVALID, "an f16/bf16 backward with grad_x needs an fp32 workspace of %lld bytes "
                        "(dcn_backward_ws)", (long long)need);
        if ((int64_t)workspace_bytes < need)
            return fail(DCN_ERR_INVALID, "workspace has %zu bytes, %lld needed", workspace_bytes, (long long)need);
        if ((uintptr_t)workspace % 4) return fail(DCN_ERR_UNSUPPORTED, "workspace is not aligned to 4 bytes");
    }
    if (!grad_x && !grad_offset && !grad_mask) return ok();
    return hip_status(dcn::launch_dcn_backward(G, desc->dtype, x, offset, mask, grad_out, grad_x, grad_offset,
                                               grad_mask, need > 0 ? (float*)workspace : nullptr,
                                               (hipStream_t)stream));
}

dcn_status dcn_backward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                        const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask, void* stream)
{
    return backward_impl(desc, x, offset, mask, grad_out, grad_x, grad_offset, grad_mask, nullptr, 0, stream);
}

dcn_status dcn_backward_workspace_size(const dcn_desc* desc, size_t* bytes)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    if (!bytes) return fail(DCN_ERR_INVALID, "bytes is NULL");
    *bytes = (size_t)backward_ws_bytes(desc);
    return ok();
}

dcn_status dcn_backward_ws(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                           const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    return backward_impl(desc, x, offset, mask, grad_out, grad_x, grad_offset, grad_mask, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch for dcn_backward_noalloc: the fp32 sums of an f16/bf16 grad_x, in a
// device array the library owns (one copy per GPU, held until the process
// ends).  Host code never uses the array's name as an address: its device
// address is looked up once per device with hipGetSymbolAddress and kept.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device and kept (concurrent first calls store the same address).
dcn_status scratch_ptr(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DCN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DCN_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev, kMaxDevices);
    void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(DCN_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
    }
    *out = p;
    return DCN_OK;
}

}  // namespace

extern "C" {

dcn_status dcn_backward_noalloc(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask, void* stream)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    if ((st = check_backward_ptrs(desc, x, offset, mask, grad_out, grad_x, grad_offset, grad_mask))) return st;
    const int64_t need = grad_x ? backward_ws_bytes(desc) : 0;
    if (need > (int64_t)kScratchBytes)
        return fail(DCN_ERR_INVALID, "dcn_backward_noalloc: grad_x needs %lld bytes of fp32 sums, more than the "
                    "%zu bytes of its static scratch (use dcn_backward_ws)", (long long)need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (st = scratch_ptr(&ws)) != DCN_OK) return st;
    return backward_impl(desc, x, offset, mask, grad_out, grad_x, grad_offset, grad_mask, ws,
                         need > 0 ? kScratchBytes : 0, stream);
}

dcn_status dcn_offset_mask(const dcn_desc* desc, const void* x, const void* dw_weight, const void* dw_bias,
                           const void* om_weight, const void* om_bias, void* offset, void* mask, void* stream)
{
    dcn::Geom G;
    dcn_status st = make_geom(desc, &G);
    if (st != DCN_OK) return st;
    if (G.ho != G.h || G.wo != G.w)
        return fail(DCN_ERR_UNSUPPORTED, "dcn_offset_mask needs an output the size of the input (stride 1, "
                    "(kernel-1)*dil == 2*pad)");
    if (desc->dtype == DCN_F32) return fail(DCN_ERR_UNSUPPORTED, "dcn_offset_mask supports f16 and bf16");
    if (G.c % 8) return fail(DCN_ERR_UNSUPPORTED, "dcn_offset_mask needs c %% 8 == 0");
    if ((st = check_ptr(x, "x", 16)) || (st = check_ptr(dw_weight, "dw_weight", 16)) ||
        (st = check_ptr(dw_bias, "dw_bias", 16)) || (st = check_ptr(om_weight, "om_weight", 16)) ||
        (st = check_ptr(om_bias, "om_bias", 2)) || (st = check_ptr(offset, "offset", 16)) ||
        (st = check_ptr(mask, "mask", 16)))
        return st;
    if ((int64_t)G.c * G.g * G.K * 3 >= kMaxElems) return fail(DCN_ERR_INVALID, "an element count reaches 2^31");
    int lds_limit = 65536, num_cus = 256;
    dcn::device_limits(&lds_limit, &num_cus);
    if (!dcn::frontend_supported(G, desc->dtype, lds_limit))
        return fail(DCN_ERR_UNSUPPORTED, "c and group*K*3 are too large for the LDS tiles");
    return hip_status(dcn::launch_dcn_offset_mask(G, desc->dtype, x, dw_weight, dw_bias, om_weight, om_bias, offset,
                                                  mask, (hipStream_t)stream));
}

// Validation shared by the MSDA entry points; fills G on success.
static dcn_status msda_geom(const msda_desc* d, const int32_t* shapes, dcn::MsdaGeom& G)
{
    if (!d) return fail(DCN_ERR_INVALID, "desc is NULL");
    if (d->n < 1 || d->len_q < 1 || d->heads < 1 || d->head_dim < 1 || d->levels < 1 || d->points < 1)
        return fail(DCN_ERR_INVALID, "n, len_q, heads, head_dim, levels and points must be >= 1");
    if (d->softmax != 0 && d->softmax != 1) return fail(DCN_ERR_INVALID, "softmax must be 0 or 1");
    if (d->dtype != DCN_F32 && d->dtype != DCN_F16 && d->dtype != DCN_BF16)
        return fail(DCN_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (!shapes) return fail(DCN_ERR_INVALID, "spatial_shapes is NULL");
    if (d->levels > dcn::MSDA_MAX_LEVELS)
        return fail(DCN_ERR_UNSUPPORTED, "at most %d levels are supported", dcn::MSDA_MAX_LEVELS);
    G.n = d->n; G.q = d->len_q; G.m = d->heads; G.dh = d->head_dim; G.L = d->levels; G.P = d->points;
    G.softmax = d->softmax;
    G.half_inv_p = 0.5 / d->points;
    int64_t S = 0;
    for (int l = 0; l < d->levels; ++l) {
        const int32_t hl = shapes[2 * l], wl = shapes[2 * l + 1];
        if (hl < 1 || wl < 1 || hl >= kMaxSide || wl >= kMaxSide)
            return fail(DCN_ERR_INVALID, "level %d has an invalid shape (%d, %d)", l, hl, wl);
        G.H[l] = hl;
        G.W[l] = wl;
        G.inv_w[l] = 1.0 / wl;
        G.inv_h[l] = 1.0 / hl;
        G.start[l] = (int)S;
        S += (int64_t)hl * wl;
        if (S >= kMaxElems) return fail(DCN_ERR_INVALID, "an element count reaches 2^31");
    }
    const int64_t LP = (int64_t)d->levels * d->points;
    const int64_t nq = (int64_t)d->n * d->len_q * d->heads;
    if ((int64_t)d->n * S * d->heads * d->head_dim >= kMaxElems || nq * LP * 2 >= kMaxElems ||
        nq * d->head_dim >= kMaxElems)
        return fail(DCN_ERR_INVALID, "an element count reaches 2^31");
    G.S = (int)S;
    return DCN_OK;
}

dcn_status msda_forward(const msda_desc* d, const int32_t* shapes, const void* value, const void* loc,
                        const void* attn, void* out, void* stream)
{
    dcn::MsdaGeom G;
    dcn_status st = msda_geom(d, shapes, G);
    if (st) return st;
    if (!value || !loc || !attn || !out) return fail(DCN_ERR_INVALID, "value, loc, attn and out must not be NULL");
    if (d->dtype != DCN_F32) return fail(DCN_ERR_UNSUPPORTED, "msda_forward supports f32 only");
    if ((st = check_ptr(value, "value", 4)) || (st = check_ptr(loc, "loc", 4)) || (st = check_ptr(attn, "attn", 4)) ||
        (st = check_ptr(out, "out", 4)))
        return st;
    return hip_status(dcn::launch_msda_forward(G, (const float*)value, (const float*)loc, (const float*)attn,
                                               (float*)out, (hipStream_t)stream));
}

dcn_status msda_forward_ref(const msda_desc* d, const int32_t* shapes, int32_t ref_dims, const void* value,
                            const void* reference, const void* valid_ratios, const void* offsets, const void* attn,
                            const uint8_t* padding_mask, void* out, void* stream)
{
    dcn::MsdaGeom G;
    dcn_status st = msda_geom(d, shapes, G);
    if (st) return st;
    if (ref_dims != 2 && ref_dims != 4) return fail(DCN_ERR_INVALID, "ref_dims must be 2 or 4 (got %d)", ref_dims);
    if (!value || !reference || !offsets || !attn || !out)
        return fail(DCN_ERR_INVALID, "value, reference, offsets, attn and out must not be NULL");
    if (d->dtype != DCN_F32) return fail(DCN_ERR_UNSUPPORTED, "msda_forward_ref supports f32 only");
    if ((int64_t)d->n * d->len_q * ref_dims >= kMaxElems) return fail(DCN_ERR_INVALID, "an element count reaches 2^31");
    if ((st = check_ptr(value, "value", 4)) || (st = check_ptr(reference, "reference", 4)) ||
        (st = check_ptr(offsets, "offsets", 4)) || (st = check_ptr(attn, "attn", 4)) || (st = check_ptr(out, "out", 4)))
        return st;
    if (valid_ratios && (uintptr_t)valid_ratios % 4) return fail(DCN_ERR_UNSUPPORTED, "valid_ratios is not aligned");
    return hip_status(dcn::launch_msda_forward_ref(G, ref_dims, (const float*)value, (const float*)reference,
                                                   (const float*)valid_ratios, (const float*)offsets,
                                                   (const float*)attn, padding_mask, (float*)out,
                                                   (hipStream_t)stream));
}

static dcn_status msda_backward_impl(const msda_desc* d, const int32_t* shapes, const void* value, const void* loc,
                                     const void* attn, const void* grad_out, void* grad_value, void* grad_loc,
                                     void* grad_attn, void* workspace, size_t workspace_bytes, bool with_ws,
                                     void* stream)
{
    dcn::MsdaGeom G;
    dcn_status st = msda_geom(d, shapes, G);
    if (st) return st;
    if (!value || !loc || !attn || !grad_out)
        return fail(DCN_ERR_INVALID, "value, loc, attn and grad_out must not be NULL");
    if (d->dtype != DCN_F32) return fail(DCN_ERR_UNSUPPORTED, "msda_backward supports f32 only");
    if ((st = check_ptr(value, "value", 4)) || (st = check_ptr(loc, "loc", 4)) || (st = check_ptr(attn, "attn", 4)) ||
        (st = check_ptr(grad_out, "grad_out", 4)))
        return st;
    if (grad_value && (st = check_ptr(grad_value, "grad_value", 4))) return st;
    if (grad_loc && (st = check_ptr(grad_loc, "grad_loc", 4))) return st;
    if (grad_attn && (st = check_ptr(grad_attn, "grad_attn", 4))) return st;
    size_t need = 0;
    if (with_ws && grad_value) {
        need = dcn::msda_backward_workspace(G);
        if (need) {
            if (!workspace)
                return fail(DCN_ERR_INVALID, "msda_backward_ws with grad_value needs a workspace of %zu bytes", need);
            if (workspace_bytes < need)
                return fail(DCN_ERR_INVALID, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
            if ((uintptr_t)workspace % 256) return fail(DCN_ERR_UNSUPPORTED, "workspace is not aligned to 256 bytes");
        }
    }
    if (!grad_value && !grad_loc && !grad_attn) return ok();
    return hip_status(dcn::launch_msda_backward(G, (const float*)value, (const float*)loc, (const float*)attn,
                                                (const float*)grad_out, (float*)grad_value, (float*)grad_loc,
                                                (float*)grad_attn, need ? workspace : nullptr, need,
                                                (hipStream_t)stream));
}

dcn_status msda_backward(const msda_desc* d, const int32_t* shapes, const void* value, const void* loc,
                         const void* attn, const void* grad_out, void* grad_value, void* grad_loc, void* grad_attn,
                         void* stream)
{
    return msda_backward_impl(d, shapes, value, loc, attn, grad_out, grad_value, grad_loc, grad_attn, nullptr, 0,
                              false, stream);
}

dcn_status msda_backward_workspace_size(const msda_desc* d, const int32_t* shapes, size_t* bytes)
{
    if (!bytes) return fail(DCN_ERR_INVALID, "bytes is NULL");
    dcn::MsdaGeom G;
    dcn_status st = msda_geom(d, shapes, G);
    if (st) return st;
    *bytes = d->dtype == DCN_F32 ? dcn::msda_backward_workspace(G) : 0;
    return ok();
}

dcn_status msda_backward_ws(const msda_desc* d, const int32_t* shapes, const void* value, const void* loc,
                            const void* attn, const void* grad_out, void* grad_value, void* grad_loc, void* grad_attn,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    return msda_backward_impl(d, shapes, value, loc, attn, grad_out, grad_value, grad_loc, grad_attn, workspace,
                              workspace_bytes, true, stream);
}

#ifdef DCN_COUNT_WRITES
dcn_status dcn_debug_count_writes(unsigned int* counts, const void* out, size_t n, int dtype)
{
    if (dtype != DCN_F32 && dtype != DCN_F16 && dtype != DCN_BF16)
        return fail(DCN_ERR_INVALID, "dcn_debug_count_writes: bad dtype %d", dtype);
    if (counts && !out) return fail(DCN_ERR_INVALID, "dcn_debug_count_writes: NULL out");
    const unsigned int es = dtype == DCN_F32 ? 4u : 2u;
    hipError_t e = dcn::ring_count_writes(counts, out, n, es);
    if (e == hipSuccess) e = dcn::fwd_count_writes(counts, out, n, es);
    if (e == hipSuccess) e = dcn::msda_count_writes(counts, out, n, es);
    if (e == hipSuccess) e = dcn::frontend_count_writes(counts, out, n, es);
    return hip_status(e);
}
#endif

}  // extern "C"
