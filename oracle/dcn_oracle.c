/*
 * dcn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU statement, in double precision, of what
 * the deformable sampling operators compute.  Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark load it.  The product library
 * never links, loads or calls it, and the two share no code: no header, no
 * helper, no table.  Inputs arrive as doubles that hold the exact stored
 * values (f16/bf16/f32 all convert to double without rounding).
 *
 * Sources, cited by page title and section:
 *  [IIM]   "InternImage: Deformable Convolutions at Scale"
 *          Ch.1 "From Convolution to Deformable": the regular tap grid R and a
 *               learned offset added per tap.
 *          Ch.2 "Deformable Sampling & Bilinear Reads": x0 = floor(px),
 *               a = px - x0, corner weights (1-a)(1-b), a(1-b), (1-a)b, ab,
 *               a corner outside the map reads zero.
 *          Ch.3 "The DCNv3 Operator": modulations softmax-normalised over the
 *               K taps (max subtracted first).
 *          Ch.4 "Groups & Weight Sharing": C split into G groups of C/G
 *               channels; each group has its own K offsets and K modulations.
 *  [V4]    "DCNv4: Unbounded Weights"
 *          "Why Is Sampling Just 9 Points Still Slow?": the per-group sum
 *               y_g(p0) = sum_k m_gk x_g(p0 + p_k + dp_gk).
 *          "1. Remove Softmax": DCNv4 uses m as given (any real value).
 *  [DDETR] "Deformable DETR: Learn Where to Read"
 *          "A learned location can fall between cells": pixel coordinates
 *               x = u*W - 1/2, y = v*H - 1/2, tent weights (1-|x-i|)+(1-|y-j|)+,
 *               zero outside, no clamping and no renormalisation.
 *          "Mix samples with a per-head budget": one softmax per head over all
 *               levels and points jointly; the head output is the weighted sum.
 *          "From the equations to runnable arithmetic", rows 2 and 3.
 *
 * Readings where the pages leave a step open (each one is a convention that
 * the product path follows too):
 *  - Tap order: the grid R is listed with the second (y) component varying
 *    fastest, so tap k sits at kx = k / kernel_h, ky = k % kernel_h.
 *  - The offset pair of a tap is stored (dx, dy): x is the column.
 *  - Stride, padding and dilation follow ordinary convolution geometry:
 *    px = wo*stride_w - pad_w + kx*dil_w + s*dx, likewise py; at a 3x3 kernel
 *    with stride 1, pad 1, dilation 1 this is exactly p0 + p_k + dp_k.
 *  - offset_scale s multiplies the stored offset before it is added.
 *  - The core sum carries no depthwise weight: the example weight w = 1 in
 *    [IIM] Ch.3 belongs to the projections around the operator.
 *  - A sample whose every corner lies outside the map contributes zero; the
 *    oracle tests that before converting coordinates to integers.  Non-finite
 *    offsets are outside the method; they are treated the same way.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Geometry and options of one DCN call.  x is [n][h][w][c]; offset is
 * [n][ho][wo][group][K][2] holding (dx, dy); mask is [n][ho][wo][group][K];
 * out is [n][ho][wo][c].  K = kernel_h * kernel_w, D = c / group. */
typedef struct {
    int n, h, w, c, group;
    int kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
    double offset_scale;
    int softmax; /* 1: mask holds logits, softmax over the K taps (DCNv3) */
} odcn_t;

/* Ordinary convolution output size. */
int oracle_dcn_out_size(const odcn_t* p, int* ho, int* wo)
{
    int eh = p->dil_h * (p->kernel_h - 1) + 1;
    int ew = p->dil_w * (p->kernel_w - 1) + 1;
    *ho = (p->h + 2 * p->pad_h - eh) / p->stride_h + 1;
    *wo = (p->w + 2 * p->pad_w - ew) / p->stride_w + 1;
    return (*ho > 0 && *wo > 0) ? 0 : 1;
}

/* Value of channel ch of one image xi ([h][w][c]) at integer (row, col),
 * zero outside the map ([IIM] Ch.2). */
static double pixel_or_zero(const double* xi, int h, int w, int c, int row, int col, int ch)
{
    if (row < 0 || row >= h || col < 0 || col >= w) return 0.0;
    return xi[((size_t)row * w + col) * c + ch];
}

/* Bilinear read at the fractional point (px, py) ([IIM] Ch.2): the four
 * corners of the unit cell around p, each weighted by the area of the
 * opposite sub-rectangle. */
static double bilinear(const double* xi, int h, int w, int c, int ch, double px, double py)
{
    if (!(px > -1.0 && px < (double)w && py > -1.0 && py < (double)h)) return 0.0;
    double fx = floor(px), fy = floor(py);
    int x0 = (int)fx, y0 = (int)fy;
    double a = px - fx, b = py - fy;
    return (1.0 - a) * (1.0 - b) * pixel_or_zero(xi, h, w, c, y0, x0, ch)
         + a * (1.0 - b) * pixel_or_zero(xi, h, w, c, y0, x0 + 1, ch)
         + (1.0 - a) * b * pixel_or_zero(xi, h, w, c, y0 + 1, x0, ch)
         + a * b * pixel_or_zero(xi, h, w, c, y0 + 1, x0 + 1, ch);
}

/* Modulation of the K taps of one (pixel, group): softmax over K with the
 * maximum subtracted ([IIM] Ch.3) or the values as given ([V4] "1. Remove
 * Softmax"). */
static void modulation(const double* raw, int K, int softmax, double* m)
{
    if (!softmax) {
        for (int k = 0; k < K; ++k) m[k] = raw[k];
        return;
    }
    double mx = raw[0];
    for (int k = 1; k < K; ++k) if (raw[k] > mx) mx = raw[k];
    double s = 0.0;
    for (int k = 0; k < K; ++k) { m[k] = exp(raw[k] - mx); s += m[k]; }
    for (int k = 0; k < K; ++k) m[k] /= s;
}

/* Sampling point of tap k for output pixel (ho, wo). */
static void tap_point(const odcn_t* p, int ho, int wo, int k, const double* off2, double* px, double* py)
{
    int kx = k / p->kernel_h, ky = k % p->kernel_h;
    *px = (double)(wo * p->stride_w - p->pad_w + kx * p->dil_w) + p->offset_scale * off2[0];
    *py = (double)(ho * p->stride_h - p->pad_h + ky * p->dil_h) + p->offset_scale * off2[1];
}

/* DCN forward: y_g(p0) = sum_k m_gk x_g(p0 + p_k + dp_gk), per group
 * ([V4] "Why Is Sampling Just 9 Points Still Slow?", [IIM] Ch.3-4). */
int oracle_dcn_forward(const odcn_t* p, const double* x, const double* offset,
                       const double* mask, double* out)
{
    int ho_n, wo_n;
    if (oracle_dcn_out_size(p, &ho_n, &wo_n)) return 1;
    const int K = p->kernel_h * p->kernel_w, G = p->group, D = p->c / p->group;
    double* m = (double*)malloc(sizeof(double) * K);
    for (int n = 0; n < p->n; ++n) {
        const double* xi = x + (size_t)n * p->h * p->w * p->c;
        for (int ho = 0; ho < ho_n; ++ho)
            for (int wo = 0; wo < wo_n; ++wo)
                for (int g = 0; g < G; ++g) {
                    size_t item = (((size_t)n * ho_n + ho) * wo_n + wo) * G + g;
                    modulation(mask + item * K, K, p->softmax, m);
                    double* o = out + (((size_t)n * ho_n + ho) * wo_n + wo) * p->c + (size_t)g * D;
                    for (int d = 0; d < D; ++d) o[d] = 0.0;
                    for (int k = 0; k < K; ++k) {
                        double px, py;
                        tap_point(p, ho, wo, k, offset + (item * K + k) * 2, &px, &py);
                        for (int d = 0; d < D; ++d)
                            o[d] += m[k] * bilinear(xi, p->h, p->w, p->c, g * D + d, px, py);
                    }
                }
    }
    free(m);
    return 0;
}

/* The same forward written with the tent form of the bilinear read
 * ([DDETR] "A learned location can fall between cells"): every pixel of the
 * map contributes (1-|px-col|)+ (1-|py-row|)+ times its value.  It shares no
 * step with bilinear() above and serves as an independent brute-force check
 * on tiny inputs. */
int oracle_dcn_forward_tent(const odcn_t* p, const double* x, const double* offset,
                            const double* mask, double* out)
{
    int ho_n, wo_n;
    if (oracle_dcn_out_size(p, &ho_n, &wo_n)) return 1;
    const int K = p->kernel_h * p->kernel_w, G = p->group, D = p->c / p->group;
    double* m = (double*)malloc(sizeof(double) * K);
    for (int n = 0; n < p->n; ++n)
        for (int ho = 0; ho < ho_n; ++ho)
            for (int wo = 0; wo < wo_n; ++wo)
                for (int g = 0; g < G; ++g) {
                    size_t item = (((size_t)n * ho_n + ho) * wo_n + wo) * G + g;
                    modulation(mask + item * K, K, p->softmax, m);
                    for (int d = 0; d < D; ++d) {
                        double acc = 0.0;
                        for (int k = 0; k < K; ++k) {
                            double px, py;
                            tap_point(p, ho, wo, k, offset + (item * K + k) * 2, &px, &py);
                            for (int row = 0; row < p->h; ++row) {
                                double ty = 1.0 - fabs(py - row);
                                if (!(ty > 0.0)) continue;
                                for (int col = 0; col < p->w; ++col) {
                                    double tx = 1.0 - fabs(px - col);
                                    if (!(tx > 0.0)) continue;
                                    acc += m[k] * tx * ty *
                                           x[(((size_t)n * p->h + row) * p->w + col) * p->c + g * D + d];
                                }
                            }
                        }
                        out[(((size_t)n * ho_n + ho) * wo_n + wo) * p->c + g * D + d] = acc;
                    }
                }
    free(m);
    return 0;
}

/* DCN backward: the analytic derivative of oracle_dcn_forward.  The pages
 * only state that the bilinear read is differentiable almost everywhere
 * ([IIM] Ch.2 "Why bilinear, and why it is differentiable"); the terms are
 * the product rule applied to the corner weights:
 *   v_k,c        = sum over corners of weight * X           (sampled value)
 *   dL/dX_corner += m_k * weight * g_c
 *   dL/dm_k      = sum_c g_c v_k,c
 *   dL/ddx_k     = s m_k sum_c g_c [(1-b)(X01 - X00) + b(X11 - X10)]
 *   dL/ddy_k     = s m_k sum_c g_c [(1-a)(X10 - X00) + a(X11 - X01)]
 * where X_rc is the corner at row y0+r, column x0+c, and with softmax
 *   dL/dz_k = m_k (dL/dm_k - sum_j m_j dL/dm_j).
 * At an integer coordinate the floor cell's (right-hand) derivative is
 * taken.  grad_x is overwritten (zeroed first).  Any grad pointer may be
 * NULL to skip that output. */
int oracle_dcn_backward(const odcn_t* p, const double* x, const double* offset,
                        const double* mask, const double* grad_out, double* grad_x,
                        double* grad_offset, double* grad_mask)
{
    int ho_n, wo_n;
    if (oracle_dcn_out_size(p, &ho_n, &wo_n)) return 1;
    const int K = p->kernel_h * p->kernel_w, G = p->group, D = p->c / p->group;
    const int H = p->h, W = p->w, C = p->c;
    double* m = (double*)malloc(sizeof(double) * K);
    double* dm = (double*)malloc(sizeof(double) * K);
    if (grad_x) memset(grad_x, 0, sizeof(double) * (size_t)p->n * H * W * C);
    for (int n = 0; n < p->n; ++n) {
        const double* xi = x + (size_t)n * H * W * C;
        double* gxi = grad_x ? grad_x + (size_t)n * H * W * C : NULL;
        for (int ho = 0; ho < ho_n; ++ho)
            for (int wo = 0; wo < wo_n; ++wo)
                for (int g = 0; g < G; ++g) {
                    size_t item = (((size_t)n * ho_n + ho) * wo_n + wo) * G + g;
                    modulation(mask + item * K, K, p->softmax, m);
                    const double* go = grad_out + (((size_t)n * ho_n + ho) * wo_n + wo) * C + (size_t)g * D;
                    for (int k = 0; k < K; ++k) {
                        double px, py;
                        tap_point(p, ho, wo, k, offset + (item * K + k) * 2, &px, &py);
                        double gdx = 0.0, gdy = 0.0, gm = 0.0;
                        if (px > -1.0 && px < (double)W && py > -1.0 && py < (double)H) {
                            double fx = floor(px), fy = floor(py);
                            int x0 = (int)fx, y0 = (int)fy;
                            double a = px - fx, b = py - fy;
                            for (int d = 0; d < D; ++d) {
                                int ch = g * D + d;
                                double X00 = pixel_or_zero(xi, H, W, C, y0, x0, ch);
                                double X01 = pixel_or_zero(xi, H, W, C, y0, x0 + 1, ch);
                                double X10 = pixel_or_zero(xi, H, W, C, y0 + 1, x0, ch);
                                double X11 = pixel_or_zero(xi, H, W, C, y0 + 1, x0 + 1, ch);
                                double v = (1 - a) * (1 - b) * X00 + a * (1 - b) * X01
                                         + (1 - a) * b * X10 + a * b * X11;
                                gm += go[d] * v;
                                gdx += go[d] * ((1 - b) * (X01 - X00) + b * (X11 - X10));
                                gdy += go[d] * ((1 - a) * (X10 - X00) + a * (X11 - X01));
                                if (gxi) {
                                    double wgt[4] = {(1 - a) * (1 - b), a * (1 - b), (1 - a) * b, a * b};
                                    int rr[4] = {y0, y0, y0 + 1, y0 + 1};
                                    int cc[4] = {x0, x0 + 1, x0, x0 + 1};
                                    for (int q = 0; q < 4; ++q)
                                        if (rr[q] >= 0 && rr[q] < H && cc[q] >= 0 && cc[q] < W)
                                            gxi[((size_t)rr[q] * W + cc[q]) * C + ch] += m[k] * wgt[q] * go[d];
                                }
                            }
                        }
                        dm[k] = gm;
                        if (grad_offset) {
                            grad_offset[(item * K + k) * 2 + 0] = p->offset_scale * m[k] * gdx;
                            grad_offset[(item * K + k) * 2 + 1] = p->offset_scale * m[k] * gdy;
                        }
                    }
                    if (grad_mask) {
                        if (p->softmax) {
                            double s = 0.0;
                            for (int k = 0; k < K; ++k) s += m[k] * dm[k];
                            for (int k = 0; k < K; ++k) grad_mask[item * K + k] = m[k] * (dm[k] - s);
                        } else {
                            for (int k = 0; k < K; ++k) grad_mask[item * K + k] = dm[k];
                        }
                    }
                }
    }
    free(m);
    free(dm);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Multi-scale deformable attention ([DDETR]).                               */
/* value is [n][S][heads][head_dim] with the levels flattened level-major,   */
/* row-major inside a level (S = sum_l H_l W_l); shapes[l] = (H_l, W_l);     */
/* loc is [n][len_q][heads][levels][points][2] holding normalised (u, v),    */
/* u along the width; attn is [n][len_q][heads][levels][points]; out is      */
/* [n][len_q][heads][head_dim].                                              */

typedef struct {
    int n, len_q, heads, head_dim, levels, points;
    int softmax; /* 1: attn holds logits, one softmax per head over all levels*points */
} omsda_t;

/* Joint softmax over the L*P logits of one head, maximum subtracted
 * ([DDETR] "Mix samples with a per-head budget"), or the weights as given. */
static void head_weights(const double* raw, int LP, int softmax, double* A)
{
    modulation(raw, LP, softmax, A);
}

/* Start of each level in the flattened value tensor. */
static size_t level_start(const int* shapes, int l)
{
    size_t s = 0;
    for (int i = 0; i < l; ++i) s += (size_t)shapes[2 * i] * shapes[2 * i + 1];
    return s;
}

/* Bilinear read of channel d of head h at normalised (u, v) of one level:
 * x = u*W - 1/2, y = v*H - 1/2, the four neighbours of (x, y) with tent
 * weights, zero outside ([DDETR] "A learned location can fall between
 * cells").  vl points at the level's first position of image n. */
static double level_read(const double* vl, int Hl, int Wl, int heads, int dh, int h, int d,
                         double u, double v)
{
    double x = u * Wl - 0.5, y = v * Hl - 0.5;
    if (!(x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl)) return 0.0;
    int x0 = (int)floor(x), y0 = (int)floor(y);
    double total = 0.0;
    for (int row = y0; row <= y0 + 1; ++row)
        for (int col = x0; col <= x0 + 1; ++col) {
            double wt = (1.0 - fabs(x - col)) * (1.0 - fabs(y - row));
            if (row >= 0 && row < Hl && col >= 0 && col < Wl)
                total += wt * vl[(((size_t)row * Wl + col) * heads + h) * dh + d];
        }
    return total;
}

int oracle_msda_forward(const omsda_t* p, const int* shapes, const double* value,
                        const double* loc, const double* attn, double* out)
{
    const int L = p->levels, P = p->points, M = p->heads, Dh = p->head_dim;
    const size_t S = level_start(shapes, L);
    double* A = (double*)malloc(sizeof(double) * L * P);
    for (int n = 0; n < p->n; ++n)
        for (int q = 0; q < p->len_q; ++q)
            for (int h = 0; h < M; ++h) {
                size_t qh = ((size_t)n * p->len_q + q) * M + h;
                head_weights(attn + qh * L * P, L * P, p->softmax, A);
                double* o = out + qh * Dh;
                for (int d = 0; d < Dh; ++d) o[d] = 0.0;
                for (int l = 0; l < L; ++l) {
                    const double* vl = value + ((size_t)n * S + level_start(shapes, l)) * M * Dh;
                    for (int pt = 0; pt < P; ++pt) {
                        const double* uv = loc + ((qh * L + l) * P + pt) * 2;
                        for (int d = 0; d < Dh; ++d)
                            o[d] += A[l * P + pt] *
                                    level_read(vl, shapes[2 * l], shapes[2 * l + 1], M, Dh, h, d, uv[0], uv[1]);
                    }
                }
            }
    free(A);
    return 0;
}

/* Brute-force MSDA: every position of every level contributes with its tent
 * weight (the sum over all i, j written on the page).  Independent of
 * level_read(); for tiny inputs only. */
int oracle_msda_forward_tent(const omsda_t* p, const int* shapes, const double* value,
                             const double* loc, const double* attn, double* out)
{
    const int L = p->levels, P = p->points, M = p->heads, Dh = p->head_dim;
    const size_t S = level_start(shapes, L);
    double* A = (double*)malloc(sizeof(double) * L * P);
    for (int n = 0; n < p->n; ++n)
        for (int q = 0; q < p->len_q; ++q)
            for (int h = 0; h < M; ++h) {
                size_t qh = ((size_t)n * p->len_q + q) * M + h;
                head_weights(attn + qh * L * P, L * P, p->softmax, A);
                for (int d = 0; d < Dh; ++d) {
                    double acc = 0.0;
                    size_t start = 0;
                    for (int l = 0; l < L; ++l) {
                        int Hl = shapes[2 * l], Wl = shapes[2 * l + 1];
                        for (int pt = 0; pt < P; ++pt) {
                            const double* uv = loc + ((qh * L + l) * P + pt) * 2;
                            double x = uv[0] * Wl - 0.5, y = uv[1] * Hl - 0.5;
                            for (int row = 0; row < Hl; ++row) {
                                double ty = 1.0 - fabs(y - row);
                                if (!(ty > 0.0)) continue;
                                for (int col = 0; col < Wl; ++col) {
                                    double tx = 1.0 - fabs(x - col);
                                    if (!(tx > 0.0)) continue;
                                    acc += A[l * P + pt] * tx * ty *
                                           value[((((size_t)n * S + start + (size_t)row * Wl + col) * M) + h) * Dh + d];
                                }
                            }
                        }
                        start += (size_t)Hl * Wl;
                    }
                    out[qh * Dh + d] = acc;
                }
            }
    free(A);
    return 0;
}

/* MSDA backward: the derivative of oracle_msda_forward, written out.
 *
 * For one query, head and sample i (level l, point p) at pixel coordinate
 * x = u*W_l - 1/2, y = v*H_l - 1/2 with x0 = floor(x), a = x - x0 (y0, b
 * likewise), corners V_rc (row y0+r, column x0+c, zero outside) and the
 * output gradient g of that query and head ([DDETR] "A learned location can
 * fall between cells": the read is a function of the location, so it is
 * differentiable in it; "Mix samples with a per-head budget"):
 *   s_i        = (1-a)(1-b) V00 + a(1-b) V01 + (1-a) b V10 + a b V11
 *   dL/dA_i    = <g, s_i>
 *   dL/dV_rc  += A_i * (corner weight) * g            (corners inside the level)
 *   dL/du_i    = W_l * A_i * <g, (1-b)(V01-V00) + b(V11-V10)>
 *   dL/dv_i    = H_l * A_i * <g, (1-a)(V10-V00) + a(V11-V01)>
 * and, when attn holds logits z of the joint softmax A = softmax(z),
 *   dL/dz_i    = A_i (dL/dA_i - sum_j A_j dL/dA_j).
 * A sample that is outside the level (every corner outside) contributes
 * nothing and has zero location gradient.  At an integer coordinate the floor
 * cell's (right-hand) derivative is taken.  grad_value is overwritten (zeroed
 * first).  Any grad pointer may be NULL to skip that output. */
int oracle_msda_backward(const omsda_t* p, const int* shapes, const double* value,
                         const double* loc, const double* attn, const double* grad_out,
                         double* grad_value, double* grad_loc, double* grad_attn)
{
    const int L = p->levels, P = p->points, M = p->heads, Dh = p->head_dim, LP = L * P;
    const size_t S = level_start(shapes, L);
    double* A = (double*)malloc(sizeof(double) * LP);
    double* dA = (double*)malloc(sizeof(double) * LP);
    if (grad_value) memset(grad_value, 0, sizeof(double) * (size_t)p->n * S * M * Dh);
    for (int n = 0; n < p->n; ++n)
        for (int q = 0; q < p->len_q; ++q)
            for (int h = 0; h < M; ++h) {
                const size_t qh = ((size_t)n * p->len_q + q) * M + h;
                head_weights(attn + qh * LP, LP, p->softmax, A);
                const double* g = grad_out + qh * Dh;
                for (int l = 0; l < L; ++l) {
                    const int Hl = shapes[2 * l], Wl = shapes[2 * l + 1];
                    const size_t base = (size_t)n * S + level_start(shapes, l);
                    for (int pt = 0; pt < P; ++pt) {
                        const int i = l * P + pt;
                        const double* uv = loc + (qh * LP + i) * 2;
                        double du = 0.0, dv = 0.0, da_i = 0.0;
                        const double x = uv[0] * Wl - 0.5, y = uv[1] * Hl - 0.5;
                        if (x > -1.0 && x < (double)Wl && y > -1.0 && y < (double)Hl) {
                            const int x0 = (int)floor(x), y0 = (int)floor(y);
                            const double a = x - x0, b = y - y0;
                            const double wt[4] = {(1 - a) * (1 - b), a * (1 - b), (1 - a) * b, a * b};
                            for (int d = 0; d < Dh; ++d) {
                                double V[4];
                                for (int c = 0; c < 4; ++c) {
                                    const int row = y0 + c / 2, col = x0 + c % 2;
                                    const int in = row >= 0 && row < Hl && col >= 0 && col < Wl;
                                    const size_t idx = ((base + (size_t)row * Wl + col) * M + h) * Dh + d;
                                    V[c] = in ? value[idx] : 0.0;
                                    if (in && grad_value) grad_value[idx] += A[i] * wt[c] * g[d];
                                }
                                const double s = wt[0] * V[0] + wt[1] * V[1] + wt[2] * V[2] + wt[3] * V[3];
                                da_i += g[d] * s;
                                du += g[d] * ((1 - b) * (V[1] - V[0]) + b * (V[3] - V[2]));
                                dv += g[d] * ((1 - a) * (V[2] - V[0]) + a * (V[3] - V[1]));
                            }
                            du *= A[i] * Wl;
                            dv *= A[i] * Hl;
                        }
                        dA[i] = da_i;
                        if (grad_loc) {
                            grad_loc[(qh * LP + i) * 2] = du;
                            grad_loc[(qh * LP + i) * 2 + 1] = dv;
                        }
                    }
                }
                if (grad_attn) {
                    double t = 0.0;
                    if (p->softmax)
                        for (int i = 0; i < LP; ++i) t += A[i] * dA[i];
                    for (int i = 0; i < LP; ++i)
                        grad_attn[qh * LP + i] = p->softmax ? A[i] * (dA[i] - t) : dA[i];
                }
            }
    free(A);
    free(dA);
    return 0;
}
