/*
 * msda_oracle.c -- CPU oracle for the multi-scale deformable attention core.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers. The product (the HIP
 * library and its Python binding) never calls, links or shares code with
 * this file, and this file includes nothing of the product.
 *
 * Plain, single-threaded, slow on purpose: every output element is the
 * defining sum written out, accumulated in double.
 *
 * What is computed (sources are the pages on deformable attention):
 *
 *   out[b,q,m,:] = sum_l sum_k A[b,q,m,l,k] * x^l_m( phi_l(loc[b,q,m,l,k]) )
 *
 *   -- the MSDeformAttn equation of the deformable-attention tutorial
 *      (discosf.com, section 2.2), restated with the same symbols in the
 *      DETR-to-Deformable-DETR article (cf-1.com, section 3.1) and the CSDN
 *      MSDA explainer (section 2, core formula). The value projection W'_m
 *      and output projection W_m are outside the core: x^l_m is the already
 *      projected value of head m on level l.
 *
 *   phi_l maps a normalized location (u, v) to level-l pixel coordinates.
 *   Pixels are treated as cell centres (grid_sample with
 *   align_corners=False, cf-1.com section 5.3 fallback; CSDN explainer
 *   section 3, implementation note 2), so pixel i of a level of width W
 *   sits at u = (i + 0.5) / W and
 *        x = u * W - 0.5,   y = v * H - 0.5.
 *   (u is the width axis: the offset normalizer is stacked as (W, H) in
 *   cf-1.com section 3.2; spatial_shapes rows are (H, W), cf-1.com 3.3.)
 *
 *   x^l_m(x, y) is bilinear interpolation over the four integer pixels
 *   around (x, y), weighted by distance (discosf.com section 2.1 and 3.2).
 *   A pixel outside the level contributes zero: out-of-range samples are
 *   zeroed in the interpolation mask (discosf.com section 2.2) --
 *   padding_mode='zeros' in cf-1.com 5.3. Each corner is tested on its
 *   own; the remaining weights are not renormalized.
 *
 *   Backward: the derivative of the same expression. floor() is piecewise
 *   constant, so the location gradient flows through the bilinear weights
 *   only (discosf.com section 3.2). Inside a cell the derivative is the
 *   one of that cell's bilinear polynomial; at an exact integer coordinate
 *   the cell is the one floor() selects, i.e. the right-sided derivative.
 *
 * Precision: double throughout, with one exception. The coordinate map
 * decides an integer (the cell), so it is evaluated in the same precision as
 * the GPU kernel: the single-precision fused multiply-add
 * fmaf(u, (float)W, -0.5f), which C99 defines as correctly rounded. Every
 * later step (floor, fraction, weights, sums) is exact or double.
 *
 * Non-finite or huge coordinates: the corner bounds tests are written so that
 * NaN fails them; such a sample contributes nothing and gets zero gradients.
 *
 * Layouts (row-major, contiguous):
 *   value              [B, Nv, M, D]      Nv = sum_l H_l * W_l
 *   spatial_shapes     [L, 2]             rows (H_l, W_l)
 *   level_start_index  [L]                start row of level l in Nv
 *   loc                [B, Nq, M, L, K, 2] (u, v) = (x, y) normalized
 *   attn               [B, Nq, M, L, K]
 *   out, grad_out      [B, Nq, M, D]      (== [B, Nq, M*D], head-major)
 *
 * Each "abs" output, when non-NULL, receives the sum of the absolute values of
 * the terms that make up the matching result element. Tests use it to scale
 * the tolerance of a floating-point sum whose terms may cancel.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1

typedef struct {
    int valid;     /* pixel inside the level                              */
    int64_t row;   /* row in the flattened Nv axis (valid corners only)   */
    double w;      /* bilinear weight                                     */
    double dw_dx;  /* d w / d x   (x in level pixels)                     */
    double dw_dy;  /* d w / d y                                           */
} corner_t;

/* phi_l: normalized (u, v) -> level pixel coordinates, cell-centre convention. */
static void level_pixel_coords(float u, float v, int64_t H, int64_t W, double *x,
                               double *y) {
    *x = (double)fmaf(u, (float)W, -0.5f);
    *y = (double)fmaf(v, (float)H, -0.5f);
}

/* The four integer pixels around (x, y) on a level of H x W pixels whose first
 * row in the flattened axis is `start`, with their bilinear weights and the
 * derivatives of those weights. Corner order: (y0,x0), (y0,x0+1), (y0+1,x0),
 * (y0+1,x0+1). */
static void bilinear_corners(double x, double y, int64_t H, int64_t W, int64_t start,
                             corner_t c[4]) {
    const double x0 = floor(x), y0 = floor(y);
    const double fx = x - x0, fy = y - y0;
    for (int dy = 0; dy < 2; ++dy) {
        for (int dx = 0; dx < 2; ++dx) {
            corner_t *k = &c[2 * dy + dx];
            const double xc = x0 + dx, yc = y0 + dy;
            const double wx = dx ? fx : 1.0 - fx;
            const double wy = dy ? fy : 1.0 - fy;
            k->w = wx * wy;
            k->dw_dx = (dx ? 1.0 : -1.0) * wy;
            k->dw_dy = (dy ? 1.0 : -1.0) * wx;
            /* written so that NaN and +-Inf fail */
            k->valid = (xc >= 0.0) && (xc < (double)W) && (yc >= 0.0) && (yc < (double)H);
            k->row = k->valid ? start + (int64_t)yc * W + (int64_t)xc : -1;
        }
    }
}

static int check_args(int64_t B, int64_t Nv, int64_t M, int64_t D, int64_t L, int64_t Nq,
                      int64_t K, const int64_t *shapes, const int64_t *lsi) {
    if (B < 0 || Nv < 0 || M < 0 || D < 0 || L < 0 || Nq < 0 || K < 0) return ORACLE_BAD_ARGS;
    if (!shapes || !lsi) return L == 0 ? ORACLE_OK : ORACLE_BAD_ARGS;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        if (shapes[2 * l] < 1 || shapes[2 * l + 1] < 1) return ORACLE_BAD_ARGS;
        if (lsi[l] != total) return ORACLE_BAD_ARGS;
        total += shapes[2 * l] * shapes[2 * l + 1];
    }
    return total == Nv ? ORACLE_OK : ORACLE_BAD_ARGS;
}

/* Forward. out[b,q,m,d] = sum_{l,k,c valid} A * w_c * value[b, row_c, m, d]. */
int msda_oracle_forward(int64_t B, int64_t Nv, int64_t M, int64_t D, int64_t L, int64_t Nq,
                        int64_t K, const double *value, const int64_t *shapes,
                        const int64_t *lsi, const float *loc, const double *attn, double *out,
                        double *out_abs) {
    if (check_args(B, Nv, M, D, L, Nq, K, shapes, lsi) != ORACLE_OK) return ORACLE_BAD_ARGS;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int64_t m = 0; m < M; ++m) {
                double *o = out + ((b * Nq + q) * M + m) * D;
                double *oa = out_abs ? out_abs + ((b * Nq + q) * M + m) * D : NULL;
                for (int64_t d = 0; d < D; ++d) {
                    o[d] = 0.0;
                    if (oa) oa[d] = 0.0;
                }
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t p = (((b * Nq + q) * M + m) * L + l) * K + k;
                        const double a = attn[p];
                        double x, y;
                        corner_t c[4];
                        level_pixel_coords(loc[2 * p], loc[2 * p + 1], H, W, &x, &y);
                        bilinear_corners(x, y, H, W, lsi[l], c);
                        for (int i = 0; i < 4; ++i) {
                            if (!c[i].valid) continue;
                            const double *v = value + ((b * Nv + c[i].row) * M + m) * D;
                            for (int64_t d = 0; d < D; ++d) {
                                const double t = a * c[i].w * v[d];
                                o[d] += t;
                                if (oa) oa[d] += fabs(t);
                            }
                        }
                    }
                }
            }
    return ORACLE_OK;
}

/* Backward, with g = grad_out[b,q,m,:] and s[d] = sum_c w_c * v_c[d] the
 * bilinear sample of one point:
 *   grad_attn[b,q,m,l,k]      = sum_d g[d] * s[d]
 *   grad_loc[b,q,m,l,k,0]     = A * sum_d g[d] * ds[d]/dx * dx/du,  dx/du = W
 *   grad_loc[b,q,m,l,k,1]     = A * sum_d g[d] * ds[d]/dy * dy/dv,  dy/dv = H
 *   grad_value[b,row_c,m,d]  += A * w_c * g[d]          (valid corners only)
 * Any of the three gradient pointers may be NULL (that gradient is skipped);
 * each abs pointer may be NULL. grad_value is overwritten (zeroed first). */
int msda_oracle_backward(int64_t B, int64_t Nv, int64_t M, int64_t D, int64_t L, int64_t Nq,
                         int64_t K, const double *value, const int64_t *shapes,
                         const int64_t *lsi, const float *loc, const double *attn,
                         const double *grad_out, double *grad_value, double *grad_loc,
                         double *grad_attn, double *grad_value_abs, double *grad_loc_abs,
                         double *grad_attn_abs) {
    if (check_args(B, Nv, M, D, L, Nq, K, shapes, lsi) != ORACLE_OK) return ORACLE_BAD_ARGS;
    const size_t nval = (size_t)(B * Nv * M * D);
    if (grad_value) memset(grad_value, 0, nval * sizeof(double));
    if (grad_value_abs) memset(grad_value_abs, 0, nval * sizeof(double));
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int64_t m = 0; m < M; ++m) {
                const double *g = grad_out + ((b * Nq + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t p = (((b * Nq + q) * M + m) * L + l) * K + k;
                        const double a = attn[p];
                        double x, y;
                        corner_t c[4];
                        level_pixel_coords(loc[2 * p], loc[2 * p + 1], H, W, &x, &y);
                        bilinear_corners(x, y, H, W, lsi[l], c);
                        double ga = 0.0, ga_abs = 0.0;
                        double gx = 0.0, gx_abs = 0.0, gy = 0.0, gy_abs = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            double s = 0.0, s_abs = 0.0;
                            double ds_dx = 0.0, dsx_abs = 0.0, ds_dy = 0.0, dsy_abs = 0.0;
                            for (int i = 0; i < 4; ++i) {
                                if (!c[i].valid) continue;
                                const double vd = value[((b * Nv + c[i].row) * M + m) * D + d];
                                s += c[i].w * vd;
                                s_abs += fabs(c[i].w * vd);
                                ds_dx += c[i].dw_dx * vd;
                                dsx_abs += fabs(c[i].dw_dx * vd);
                                ds_dy += c[i].dw_dy * vd;
                                dsy_abs += fabs(c[i].dw_dy * vd);
                            }
                            ga += g[d] * s;
                            ga_abs += fabs(g[d]) * s_abs;
                            gx += g[d] * ds_dx;
                            gx_abs += fabs(g[d]) * dsx_abs;
                            gy += g[d] * ds_dy;
                            gy_abs += fabs(g[d]) * dsy_abs;
                        }
                        if (grad_attn) grad_attn[p] = ga;
                        if (grad_attn_abs) grad_attn_abs[p] = ga_abs;
                        if (grad_loc) {
                            grad_loc[2 * p] = a * gx * (double)W;
                            grad_loc[2 * p + 1] = a * gy * (double)H;
                        }
                        if (grad_loc_abs) {
                            grad_loc_abs[2 * p] = fabs(a) * gx_abs * (double)W;
                            grad_loc_abs[2 * p + 1] = fabs(a) * gy_abs * (double)H;
                        }
                        if (grad_value || grad_value_abs) {
                            for (int i = 0; i < 4; ++i) {
                                if (!c[i].valid) continue;
                                const size_t base = (size_t)(((b * Nv + c[i].row) * M + m) * D);
                                for (int64_t d = 0; d < D; ++d) {
                                    const double t = a * c[i].w * g[d];
                                    if (grad_value) grad_value[base + d] += t;
                                    if (grad_value_abs) grad_value_abs[base + d] += fabs(t);
                                }
                            }
                        }
                    }
                }
            }
    return ORACLE_OK;
}

/*
 * Fused front-end: the two model steps the pages put right before the core
 * (DETR-to-Deformable-DETR article, cf-1.com section 3.2):
 *
 *   loc[b,q,m,l,k] = ref[b,q,l] + off[b,q,m,l,k] / (W_l, H_l)
 *       offsets in level-l pixels, the normalizer stacked as (W, H);
 *   A[b,q,m,:]     = softmax of logits[b,q,m,:] over the L*K samples of one
 *       (query, head) (cf-1.com 3.2; CSDN MSDA explainer section 3, note 3).
 *
 * Reference points come per level, [B, Nq, L, 2] (x, y) normalized; a caller
 * with one point per query repeats it over the levels (the encoder's own
 * position on every level, discosf.com section 2.2).
 *
 * The location decides the cell, so it is formed in single precision, as the
 * GPU forms it: the quotient off / W rounded to float, then the sum rounded to
 * float. The softmax and everything after are double.
 *
 * Backward: with gLoc and gA the core's location and weight gradients,
 *   grad_off[...,0] = gLoc[...,0] / W_l,  grad_off[...,1] = gLoc[...,1] / H_l
 *   grad_ref[b,q,l] = sum over heads m and points k of gLoc[b,q,m,l,k]
 *   grad_logits[b,q,m,j] = A_j * (gA_j - sum_i A_i gA_i)   (softmax Jacobian)
 */
static float fused_coord(float ref, float off, int64_t size) {
    const float quotient = off / (float)size;
    return ref + quotient;
}

/* Locations and softmax weights of every point; NULL when out of memory. */
static int fused_front(int64_t B, int64_t M, int64_t L, int64_t Nq, int64_t K,
                       const int64_t *shapes, const float *ref, const float *off,
                       const float *logits, float **loc_out, double **attn_out) {
    const int64_t LK = L * K, T = B * Nq * M;
    float *loc = (float *)malloc((size_t)(T * LK * 2 + 1) * sizeof(float));
    double *attn = (double *)malloc((size_t)(T * LK + 1) * sizeof(double));
    if (!loc || !attn) {
        free(loc);
        free(attn);
        return ORACLE_BAD_ARGS;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int64_t m = 0; m < M; ++m) {
                const int64_t t = (b * Nq + q) * M + m;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                    const float *r = ref + ((b * Nq + q) * L + l) * 2;
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t p = t * LK + l * K + k;
                        loc[2 * p] = fused_coord(r[0], off[2 * p], W);
                        loc[2 * p + 1] = fused_coord(r[1], off[2 * p + 1], H);
                    }
                }
                const float *z = logits + t * LK;
                double zmax = -INFINITY, sum = 0.0;
                for (int64_t j = 0; j < LK; ++j) zmax = (double)z[j] > zmax ? (double)z[j] : zmax;
                for (int64_t j = 0; j < LK; ++j) sum += exp((double)z[j] - zmax);
                for (int64_t j = 0; j < LK; ++j) attn[t * LK + j] = exp((double)z[j] - zmax) / sum;
            }
    *loc_out = loc;
    *attn_out = attn;
    return ORACLE_OK;
}

int msda_oracle_forward_fused(int64_t B, int64_t Nv, int64_t M, int64_t D, int64_t L,
                              int64_t Nq, int64_t K, const double *value, const int64_t *shapes,
                              const int64_t *lsi, const float *ref, const float *off,
                              const float *logits, double *out, double *out_abs) {
    if (check_args(B, Nv, M, D, L, Nq, K, shapes, lsi) != ORACLE_OK) return ORACLE_BAD_ARGS;
    float *loc;
    double *attn;
    if (fused_front(B, M, L, Nq, K, shapes, ref, off, logits, &loc, &attn) != ORACLE_OK)
        return ORACLE_BAD_ARGS;
    const int rc = msda_oracle_forward(B, Nv, M, D, L, Nq, K, value, shapes, lsi, loc, attn, out,
                                       out_abs);
    free(loc);
    free(attn);
    return rc;
}

/* Any gradient pointer may be NULL; each abs pointer may be NULL. */
int msda_oracle_backward_fused(int64_t B, int64_t Nv, int64_t M, int64_t D, int64_t L,
                               int64_t Nq, int64_t K, const double *value, const int64_t *shapes,
                               const int64_t *lsi, const float *ref, const float *off,
                               const float *logits, const double *grad_out, double *grad_value,
                               double *grad_ref, double *grad_off, double *grad_logits,
                               double *grad_value_abs, double *grad_ref_abs,
                               double *grad_off_abs, double *grad_logits_abs) {
    if (check_args(B, Nv, M, D, L, Nq, K, shapes, lsi) != ORACLE_OK) return ORACLE_BAD_ARGS;
    const int64_t LK = L * K, T = B * Nq * M, P = T * LK;
    float *loc;
    double *attn;
    if (fused_front(B, M, L, Nq, K, shapes, ref, off, logits, &loc, &attn) != ORACLE_OK)
        return ORACLE_BAD_ARGS;
    double *gloc = (double *)malloc((size_t)(2 * P + 1) * sizeof(double));
    double *gloc_abs = (double *)malloc((size_t)(2 * P + 1) * sizeof(double));
    double *ga = (double *)malloc((size_t)(P + 1) * sizeof(double));
    double *ga_abs = (double *)malloc((size_t)(P + 1) * sizeof(double));
    int rc = (gloc && gloc_abs && ga && ga_abs) ? ORACLE_OK : ORACLE_BAD_ARGS;
    if (rc == ORACLE_OK)
        rc = msda_oracle_backward(B, Nv, M, D, L, Nq, K, value, shapes, lsi, loc, attn, grad_out,
                                  grad_value, gloc, ga, grad_value_abs, gloc_abs, ga_abs);
    if (rc == ORACLE_OK) {
        if (grad_ref) memset(grad_ref, 0, (size_t)(B * Nq * L * 2) * sizeof(double));
        if (grad_ref_abs) memset(grad_ref_abs, 0, (size_t)(B * Nq * L * 2) * sizeof(double));
        for (int64_t b = 0; b < B; ++b)
            for (int64_t q = 0; q < Nq; ++q)
                for (int64_t m = 0; m < M; ++m) {
                    const int64_t t = (b * Nq + q) * M + m;
                    double s = 0.0, s_abs = 0.0;   /* sum_i A_i gA_i */
                    for (int64_t j = 0; j < LK; ++j) {
                        s += attn[t * LK + j] * ga[t * LK + j];
                        s_abs += attn[t * LK + j] * ga_abs[t * LK + j];
                    }
                    for (int64_t l = 0; l < L; ++l) {
                        const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                        const int64_t r = ((b * Nq + q) * L + l) * 2;
                        for (int64_t k = 0; k < K; ++k) {
                            const int64_t p = t * LK + l * K + k;
                            if (grad_off) {
                                grad_off[2 * p] = gloc[2 * p] / (double)W;
                                grad_off[2 * p + 1] = gloc[2 * p + 1] / (double)H;
                            }
                            if (grad_off_abs) {
                                grad_off_abs[2 * p] = gloc_abs[2 * p] / (double)W;
                                grad_off_abs[2 * p + 1] = gloc_abs[2 * p + 1] / (double)H;
                            }
                            if (grad_ref) {
                                grad_ref[r] += gloc[2 * p];
                                grad_ref[r + 1] += gloc[2 * p + 1];
                            }
                            if (grad_ref_abs) {
                                grad_ref_abs[r] += gloc_abs[2 * p];
                                grad_ref_abs[r + 1] += gloc_abs[2 * p + 1];
                            }
                            const double a = attn[p];
                            if (grad_logits) grad_logits[p] = a * (ga[p] - s);
                            if (grad_logits_abs) grad_logits_abs[p] = a * (ga_abs[p] + s_abs);
                        }
                    }
                }
    }
    free(loc);
    free(attn);
    free(gloc);
    free(gloc_abs);
    free(ga);
    free(ga_abs);
    return rc;
}

/*
 * Grouped single-level deformable aggregation (DCNv3, deformable-attention
 * tutorial (discosf.com) section 4.2):
 *
 *   y(p0) = sum_g sum_k w_g m_gk x_g(p0 + p_k + dp_gk)
 *
 * The oracle computes the aggregation before the shared projection w_g (a
 * linear layer): for every output pixel p0 = (ho, wo), group g, grid point k,
 *
 *   out[b,ho,wo,g,:] = sum_k mask[b,ho,wo,g,k] * x_g(P)
 *   P = (wo*stride_w - pad_w + kx*dil_w + off_x,  ho*stride_h - pad_h + ky*dil_h + off_y)
 *
 * with k = ky * kernel_w + kx (p_k the dilated kernel grid; stride and
 * padding as in a convolution), P in input pixels (pixel (i, j) at x = j,
 * y = i), x_g bilinear over the four surrounding pixels with zero outside
 * the H x W input (the same interpolation as the core), and the modulation
 * scalars used as given. The page leaves the precision of P open; both sides
 * form it in single precision: the integer grid coordinate converted to
 * float (exact) plus the offset, one correctly rounded float addition.
 *
 * Layouts: input [B, H, W, G, D] (= [B, H*W, G, D]); offset
 * [B, Ho, Wo, G, K, 2] (x, y); mask [B, Ho, Wo, G, K]; out [B, Ho, Wo, G, D].
 * Backward: grad_input[b, pixel, g, :] += m * w_c * g; grad_mask = sum_d g .
 * sample; grad_off = m * sum_d g . d sample / d (x, y) (dP / d off = 1).
 */
static int dcn_check(int64_t B, int64_t H, int64_t W, int64_t G, int64_t D, int64_t kh,
                     int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                     int64_t dw, int64_t Ho, int64_t Wo) {
    if (B < 0 || H < 1 || W < 1 || G < 1 || D < 1 || kh < 1 || kw < 1 || sh < 1 || sw < 1 ||
        ph < 0 || pw < 0 || dh < 1 || dw < 1 || Ho < 0 || Wo < 0)
        return ORACLE_BAD_ARGS;
    return ORACLE_OK;
}

static void dcn_point(int64_t ho, int64_t wo, int64_t k, int64_t kw, int64_t sh, int64_t sw,
                      int64_t ph, int64_t pw, int64_t dh, int64_t dw, const float *off,
                      double *x, double *y) {
    const int64_t ky = k / kw, kx = k % kw;
    const float gx = (float)(wo * sw - pw + kx * dw);
    const float gy = (float)(ho * sh - ph + ky * dh);
    *x = (double)(float)(gx + off[0]);
    *y = (double)(float)(gy + off[1]);
}

int msda_oracle_dcn_forward(int64_t B, int64_t H, int64_t W, int64_t G, int64_t D, int64_t kh,
                            int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                            int64_t dh, int64_t dw, int64_t Ho, int64_t Wo, const double *input,
                            const float *offset, const double *mask, double *out,
                            double *out_abs) {
    if (dcn_check(B, H, W, G, D, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo) != ORACLE_OK)
        return ORACLE_BAD_ARGS;
    const int64_t K = kh * kw, Nv = H * W;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo)
                for (int64_t g = 0; g < G; ++g) {
                    const int64_t t = ((b * Ho + ho) * Wo + wo) * G + g;
                    double *o = out + t * D;
                    double *oa = out_abs ? out_abs + t * D : NULL;
                    for (int64_t d = 0; d < D; ++d) {
                        o[d] = 0.0;
                        if (oa) oa[d] = 0.0;
                    }
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t p = t * K + k;
                        double x, y;
                        corner_t c[4];
                        dcn_point(ho, wo, k, kw, sh, sw, ph, pw, dh, dw, offset + 2 * p, &x, &y);
                        bilinear_corners(x, y, H, W, 0, c);
                        const double m = mask[p];
                        for (int i = 0; i < 4; ++i) {
                            if (!c[i].valid) continue;
                            const double *v = input + ((b * Nv + c[i].row) * G + g) * D;
                            for (int64_t d = 0; d < D; ++d) {
                                const double term = m * c[i].w * v[d];
                                o[d] += term;
                                if (oa) oa[d] += fabs(term);
                            }
                        }
                    }
                }
    return ORACLE_OK;
}

int msda_oracle_dcn_backward(int64_t B, int64_t H, int64_t W, int64_t G, int64_t D, int64_t kh,
                             int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                             int64_t dh, int64_t dw, int64_t Ho, int64_t Wo, const double *input,
                             const float *offset, const double *mask, const double *grad_out,
                             double *grad_input, double *grad_offset, double *grad_mask,
                             double *grad_input_abs, double *grad_offset_abs,
                             double *grad_mask_abs) {
    if (dcn_check(B, H, W, G, D, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo) != ORACLE_OK)
        return ORACLE_BAD_ARGS;
    const int64_t K = kh * kw, Nv = H * W;
    const size_t nin = (size_t)(B * Nv * G * D);
    if (grad_input) memset(grad_input, 0, nin * sizeof(double));
    if (grad_input_abs) memset(grad_input_abs, 0, nin * sizeof(double));
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo)
                for (int64_t g = 0; g < G; ++g) {
                    const int64_t t = ((b * Ho + ho) * Wo + wo) * G + g;
                    const double *gr = grad_out + t * D;
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t p = t * K + k;
                        double x, y;
                        corner_t c[4];
                        dcn_point(ho, wo, k, kw, sh, sw, ph, pw, dh, dw, offset + 2 * p, &x, &y);
                        bilinear_corners(x, y, H, W, 0, c);
                        const double m = mask[p];
                        double gm = 0.0, gm_abs = 0.0, gx = 0.0, gx_abs = 0.0, gy = 0.0,
                               gy_abs = 0.0;
                        for (int i = 0; i < 4; ++i) {
                            if (!c[i].valid) continue;
                            const size_t base = (size_t)(((b * Nv + c[i].row) * G + g) * D);
                            for (int64_t d = 0; d < D; ++d) {
                                const double v = input[base + d];
                                gm += gr[d] * c[i].w * v;
                                gm_abs += fabs(gr[d] * c[i].w * v);
                                gx += gr[d] * c[i].dw_dx * v;
                                gx_abs += fabs(gr[d] * c[i].dw_dx * v);
                                gy += gr[d] * c[i].dw_dy * v;
                                gy_abs += fabs(gr[d] * c[i].dw_dy * v);
                                const double term = m * c[i].w * gr[d];
                                if (grad_input) grad_input[base + d] += term;
                                if (grad_input_abs) grad_input_abs[base + d] += fabs(term);
                            }
                        }
                        if (grad_mask) grad_mask[p] = gm;
                        if (grad_mask_abs) grad_mask_abs[p] = gm_abs;
                        if (grad_offset) {
                            grad_offset[2 * p] = m * gx;
                            grad_offset[2 * p + 1] = m * gy;
                        }
                        if (grad_offset_abs) {
                            grad_offset_abs[2 * p] = fabs(m) * gx_abs;
                            grad_offset_abs[2 * p + 1] = fabs(m) * gy_abs;
                        }
                    }
                }
    return ORACLE_OK;
}

/* Version tag: the loader compares it with this line of the source, so a
 * stale build cannot pass for the current one. */
int msda_oracle_version(void) { return 3; }
