/*
 * msda.h -- C ABI of the MI355X (gfx950) multi-scale deformable attention core.
 *
 * The core is the step of multi-scale deformable attention that sits between
 * the value projection and the output projection: for every query q, head m,
 * level l and point k it samples the flattened multi-level value tensor at a
 * learned location and sums the samples weighted by A_mlqk:
 *
 *   out[b,q,m,:] = sum_l sum_k A[b,q,m,l,k] * bilinear_l,m( phi_l(loc[b,q,m,l,k]) )
 *
 * Sources (pages on deformable attention):
 *   - the MSDeformAttn equation: deformable-attention tutorial (discosf.com),
 *     section 2.2; DETR-to-Deformable-DETR article (cf-1.com), section 3.1;
 *     CSDN MSDA explainer, section 2 (core formula);
 *   - phi_l, the cell-centre map of a normalized location to level pixels,
 *     x = u*W_l - 0.5, y = v*H_l - 0.5 (grid_sample with align_corners=False
 *     in the cf-1.com fallback, section 5.3; CSDN explainer section 3 note 2);
 *   - bilinear interpolation over the four surrounding pixels, with zero for
 *     pixels outside the level (discosf.com sections 2.1, 2.2 and 3.2;
 *     padding_mode 'zeros' in cf-1.com 5.3);
 *   - the flattened multi-level layout with spatial_shapes rows (H, W) and
 *     level_start_index (cf-1.com section 3.3);
 *   - the gradients of the same expression, flowing through the bilinear
 *     weights (discosf.com section 3.2).
 *
 * Layouts: dense, row-major, contiguous.
 *   value               [B, Nv, M, D]        value_dtype (fp32 or bf16)
 *   spatial_shapes      [L, 2] int64         rows (H_l, W_l)
 *   level_start_index   [L] int64            first row of level l in Nv
 *   sampling_locations  [B, Nq, M, L, K, 2]  fp32, (x, y) normalized to [0,1]
 *                                            (any value is accepted: outside
 *                                            the level reads as zero; NaN and
 *                                            Inf read as outside)
 *   attention_weights   [B, Nq, M, L, K]     fp32, used as given
 *   output, grad_output [B, Nq, M*D]         fp32, heads concatenated
 *   grad_value          [B, Nv, M, D]        fp32 (whatever value_dtype is)
 *   grad_sampling_locations [B, Nq, M, L, K, 2] fp32
 *   grad_attention_weights  [B, Nq, M, L, K]    fp32
 *
 * Ownership: every tensor pointer is a DEVICE pointer owned by the caller; a
 * pointer to a tensor with no elements may be NULL. Scratch memory, where a
 * call needs any, is a caller-provided workspace argument (except for
 * msda_backward_noalloc, whose scratch is a static device array of the
 * library). The library allocates nothing, keeps no pointer after a call
 * returns, holds no other state and may be called from several host threads. All work is enqueued
 * on `stream` (0 = the null stream) with no host synchronization; results are
 * ready when the stream reaches them. Outputs are overwritten, never
 * accumulated into.
 *
 * Errors: arguments are checked on the host before anything is enqueued; a
 * failed check launches nothing and returns MSDA_ERROR_INVALID_VALUE or
 * MSDA_ERROR_NOT_SUPPORTED. A launch failure returns MSDA_ERROR_LAUNCH.
 * The level tables live on the device and are NOT read back (that would cost
 * a synchronization): the caller guarantees H_l, W_l >= 1, sum H_l*W_l == Nv
 * and level_start_index = the prefix sums. msda_check_tables checks a host
 * copy of them.
 */
#ifndef MSDA_H_
#define MSDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSDA_VERSION_MAJOR 0
#define MSDA_VERSION_MINOR 7
#define MSDA_VERSION_PATCH 0

/* Largest number of feature levels the kernels accept. */
#define MSDA_MAX_LEVELS 16

typedef enum {
    MSDA_DTYPE_F32 = 0,  /* IEEE binary32                             */
    MSDA_DTYPE_BF16 = 1, /* bfloat16 (fp32 math)                       */
    MSDA_DTYPE_F16 = 2   /* IEEE binary16 (fp32 math)                  */
} msda_dtype_t;

typedef enum {
    MSDA_SUCCESS = 0,
    MSDA_ERROR_INVALID_VALUE = 1, /* NULL/unaligned pointer, negative or inconsistent size */
    MSDA_ERROR_NOT_SUPPORTED = 2, /* valid request outside what the kernels implement      */
    MSDA_ERROR_LAUNCH = 3,        /* the HIP runtime refused a launch                      */
    MSDA_ERROR_SCRATCH_TOO_SMALL = 4 /* msda_backward_noalloc: the problem needs more scratch
                                        than its static array holds                         */
} msda_status_t;

/* Problem sizes. B, Nq and K may be 0 (empty work; outputs are still
 * written: zeros where the sum is empty). M >= 1, L in [1, MSDA_MAX_LEVELS],
 * Nv >= 1, D in {8, 16, 32, 64}. */
typedef struct {
    int64_t B;  /* batch                       */
    int64_t Nv; /* value rows = sum H_l * W_l  */
    int64_t M;  /* heads                       */
    int64_t D;  /* channels per head           */
    int64_t L;  /* levels                      */
    int64_t Nq; /* queries                     */
    int64_t K;  /* points per head and level   */
} msda_dims_t;

/*
 * Forward: output[b,q,m*D+d] = sum_{l,k} A * sum_{corners c inside level l}
 *                              w_c * value[b, s_l + y_c*W_l + x_c, m, d]
 * computed in fp32 (bf16 values are widened exactly).
 *
 * Pointer requirements: value and output 16-byte aligned; sampling_locations
 * 8-byte aligned; the rest 4-byte aligned (int64 tables 8-byte).
 * Size limit: the value tensor must be smaller than 2 GiB (32-bit buffer
 * offsets); larger requests return MSDA_ERROR_NOT_SUPPORTED (split the batch).
 */
msda_status_t msda_forward(const msda_dims_t *dims, msda_dtype_t value_dtype,
                           const void *value, const int64_t *spatial_shapes,
                           const int64_t *level_start_index, const float *sampling_locations,
                           const float *attention_weights, float *output, hipStream_t stream);

/*
 * Backward of msda_forward for the upstream gradient grad_output:
 *   grad_attention_weights[b,q,m,l,k]  = sum_d g[d] * s[d]
 *   grad_sampling_locations[...,0]     = A * W_l * sum_d g[d] * ds[d]/dx
 *   grad_sampling_locations[...,1]     = A * H_l * sum_d g[d] * ds[d]/dy
 *   grad_value[b,row_c,m,d]            = sum over the samples whose corner c is
 *                                        that pixel of A * w_c * g[d]
 * where g = grad_output[b,q,m*D:(m+1)*D] and s is the bilinear sample. At an
 * exact integer pixel coordinate the derivative is the one of the cell that
 * floor() selects (the right-sided derivative).
 *
 * grad_value is computed without atomics: every element is written exactly
 * once (zero where no sample lands); the fp32 summation order of one element
 * may change from run to run, so its low bits may too. Any of the three
 * gradient pointers may be NULL to skip that gradient.
 *
 * workspace: device scratch owned by the caller, needed only when grad_value
 * is not NULL: at least msda_backward_workspace_size() bytes, 256-byte
 * aligned, contents irrelevant on entry and clobbered on exit. It must not be
 * used by other work until the stream has passed this call. Too small a
 * workspace returns MSDA_ERROR_INVALID_VALUE.
 *
 * Alignment: value, grad_output and grad_value 16-byte; sampling_locations
 * and grad_sampling_locations 8-byte; others 4-byte.
 * Size limit: grad_value (fp32, same shape as value) and grad_output smaller
 * than 2 GiB each.
 */
msda_status_t msda_backward(const msda_dims_t *dims, msda_dtype_t value_dtype,
                            const void *value, const int64_t *spatial_shapes,
                            const int64_t *level_start_index, const float *sampling_locations,
                            const float *attention_weights, const float *grad_output,
                            float *grad_value, float *grad_sampling_locations,
                            float *grad_attention_weights, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace msda_backward needs for these sizes (a function of the
 * sizes alone, not of the level shapes or data). Returns the same status the
 * backward's size checks would. No HIP call.
 *
 * This is the workspace of the fastest plan, which bins the points of all
 * B*M (batch, head) planes at once. A smaller workspace is accepted down to
 * msda_backward_workspace_min_size(): the value gradient then runs in passes
 * over groups of planes that share it (the results are the same, the call is
 * slower: each pass ends on its densest tiles). The fused and DCNv3 backward
 * calls follow the same rule (their workspace holds a fixed part, given by
 * their own size function minus the core's, before the planes' bins). */
msda_status_t msda_backward_workspace_size(const msda_dims_t *dims, msda_dtype_t value_dtype,
                                           size_t *bytes);

/* The smallest workspace msda_backward accepts for these sizes: the bins of
 * one (batch, head) plane per pass. No HIP call. */
msda_status_t msda_backward_workspace_min_size(const msda_dims_t *dims,
                                               msda_dtype_t value_dtype, size_t *bytes);

/* Scratch bytes the allocation-free backward holds per GPU. */
#define MSDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * msda_backward without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments (less the workspace),
 * results and errors as msda_backward; the call allocates nothing.
 *
 * Its scratch (the value gradient's binning workspace) is a static device
 * array of MSDA_NOALLOC_SCRATCH_BYTES bytes, of which each GPU the library runs on
 * holds its own copy until the process ends.
 *  - A problem whose msda_backward_workspace_size() exceeds
 *    MSDA_NOALLOC_SCRATCH_BYTES (when grad_value is requested) returns
 *    MSDA_ERROR_SCRATCH_TOO_SMALL and enqueues nothing: use msda_backward with a
 *    workspace for it.
 *  - The first call on a device looks that device's copy of the array up
 *    (hipGetSymbolAddress; no allocation). The current device must be the one
 *    `stream` belongs to.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (each call rewrites what it reads before reading it):
 *    calls that overlap on one GPU, from other streams or host threads, race
 *    and give wrong results. Order them on one stream or serialize them.
 */
msda_status_t msda_backward_noalloc(const msda_dims_t *dims, msda_dtype_t value_dtype,
                                    const void *value, const int64_t *spatial_shapes,
                                    const int64_t *level_start_index,
                                    const float *sampling_locations,
                                    const float *attention_weights, const float *grad_output,
                                    float *grad_value, float *grad_sampling_locations,
                                    float *grad_attention_weights, hipStream_t stream);

/*
 * Reduced-precision storage (guide, section 4.1 and the CSDN explainer's
 * notes on mixed precision): the tensors of the core that may be stored
 * narrower than fp32. The arithmetic stays fp32: narrow inputs are widened
 * exactly, a narrow grad_value is the fp32 result rounded to nearest even.
 *   value       F32, BF16 or F16
 *   locations   sampling_locations and attention_weights: F32 or F16
 *               (binary16 pairs (x, y) and scalars, same layouts)
 *   grad_value  the backward's value gradient: F32 or BF16
 * The location gradients stay fp32. Alignment of F16 locations 4-byte, F16
 * weights 2-byte; the rest as msda_forward / msda_backward.
 */
typedef struct {
    msda_dtype_t value;
    msda_dtype_t locations;
    msda_dtype_t grad_value;
} msda_precision_t;

/* msda_forward with the storage precisions of *precision. */
msda_status_t msda_forward_ex(const msda_dims_t *dims, const msda_precision_t *precision,
                              const void *value, const int64_t *spatial_shapes,
                              const int64_t *level_start_index, const void *sampling_locations,
                              const void *attention_weights, float *output, hipStream_t stream);

/* msda_backward with the storage precisions of *precision (workspace size as
 * msda_backward_workspace_size). */
msda_status_t msda_backward_ex(const msda_dims_t *dims, const msda_precision_t *precision,
                               const void *value, const int64_t *spatial_shapes,
                               const int64_t *level_start_index, const void *sampling_locations,
                               const void *attention_weights, const float *grad_output,
                               void *grad_value, float *grad_sampling_locations,
                               float *grad_attention_weights, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Fused front-end: the same core with its two preceding model steps done
 * inside the kernels (DETR-to-Deformable-DETR article, cf-1.com section 3.2):
 *   sampling location = reference point + offset / (W_l, H_l)
 *       offsets in level-l pixels, the normalizer stacked as (W, H);
 *   attention weights = softmax of the logits over the L*K samples of one
 *       (query, head) (also the CSDN MSDA explainer, section 3, note 3).
 * Neither the locations nor the weights are materialized in memory.
 *
 *   reference_points  [B, Nq, L, 2]        (x, y) normalized to [0, 1]; a
 *                                          point shared by the levels is
 *                                          repeated over L
 *   sampling_offsets  [B, Nq, M, L, K, 2]  (x, y) in level-l pixels, fp32
 *   attention_logits  [B, Nq, M, L*K]      fp32
 *
 * The location is formed in fp32 as ref + (off / W): the quotient and the sum
 * each correctly rounded; the core then proceeds as msda_forward does. The
 * softmax is fp32 (max-shifted exponentials).
 *
 * Alignment: value and output 16-byte; reference_points and
 * sampling_offsets 8-byte; the rest 4-byte. Sizes and errors as msda_forward.
 */
msda_status_t msda_forward_fused(const msda_dims_t *dims, msda_dtype_t value_dtype,
                                 const void *value, const int64_t *spatial_shapes,
                                 const int64_t *level_start_index, const float *reference_points,
                                 const float *sampling_offsets, const float *attention_logits,
                                 float *output, hipStream_t stream);

/*
 * Backward of msda_forward_fused for grad_output. With gLoc and gA the core's
 * location and weight gradients (see msda_backward):
 *   grad_sampling_offsets[...,0]  = gLoc[...,0] / W_l   (= A * sum_d g ds/dx)
 *   grad_sampling_offsets[...,1]  = gLoc[...,1] / H_l
 *   grad_reference_points[b,q,l]  = sum over heads m and points k of gLoc
 *   grad_attention_logits[b,q,m,j] = A_j * (gA_j - sum_i A_i gA_i)
 *   grad_value                    as msda_backward
 * Any gradient pointer may be NULL to skip it.
 *
 * workspace: at least msda_backward_fused_workspace_size() bytes, 256-byte
 * aligned, owned by the caller, clobbered; needed whenever a gradient is
 * requested and there is work (B*Nq*M > 0, or grad_value with B > 0).
 * Alignment: value, grad_output and grad_value 16-byte; reference points,
 * offsets and their gradients 8-byte; others 4-byte.
 */
msda_status_t msda_backward_fused(const msda_dims_t *dims, msda_dtype_t value_dtype,
                                  const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start_index, const float *reference_points,
                                  const float *sampling_offsets, const float *attention_logits,
                                  const float *grad_output, float *grad_value,
                                  float *grad_reference_points, float *grad_sampling_offsets,
                                  float *grad_attention_logits, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace msda_backward_fused needs for these sizes. No HIP call. */
msda_status_t msda_backward_fused_workspace_size(const msda_dims_t *dims,
                                                 msda_dtype_t value_dtype, size_t *bytes);

/*
 * Fully connected layer y = x W^T + b (torch nn.Linear semantics), fp32 on the
 * matrix cores (fp32 products, fp32 accumulation). MSDeformAttn wraps the
 * core in four of them: the value projection on the flattened input, the
 * sampling-offset and attention-weight heads on the query, and the output
 * projection (deformable-attention tutorial (discosf.com), section 3.1;
 * DETR-to-Deformable-DETR article, section 3.2).
 *
 *   x       [rows, in_features]
 *   weight  [out_features, in_features]
 *   bias    [out_features], or NULL for none
 *   y       [rows, out_features], overwritten
 *
 * rows may be 0; in_features, out_features >= 1. Sizes of 2^30 rows or 2^20
 * features and more return MSDA_ERROR_NOT_SUPPORTED. Pointers 4-byte aligned
 * (16-byte aligned tensors with feature counts that are multiples of 4 take
 * vector loads).
 */
msda_status_t msda_linear_forward(int64_t rows, int64_t in_features, int64_t out_features,
                                  const float *x, const float *weight, const float *bias,
                                  float *y, hipStream_t stream);

/*
 * Backward of msda_linear_forward for grad_y [rows, out_features]:
 *   grad_x      [rows, in_features]          = grad_y W
 *   grad_weight [out_features, in_features]  = grad_y^T x
 *   grad_bias   [out_features]               = sum of grad_y over the rows
 * each overwritten, each may be NULL to skip it. The weight and bias
 * gradients sum over the rows in a fixed order (split over blocks, then the
 * splits in order): repeatable bit for bit. workspace: at least
 * msda_linear_backward_workspace_size() bytes, 16-byte aligned, clobbered;
 * needed when grad_weight or grad_bias is requested.
 */
msda_status_t msda_linear_backward(int64_t rows, int64_t in_features, int64_t out_features,
                                   const float *x, const float *weight, const float *grad_y,
                                   float *grad_x, float *grad_weight, float *grad_bias,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace msda_linear_backward needs. No HIP call. */
msda_status_t msda_linear_backward_workspace_size(int64_t rows, int64_t in_features,
                                                  int64_t out_features, size_t *bytes);

/*
 * The whole MSDeformAttn layer around the fused core (deformable-attention
 * tutorial (discosf.com), section 3.1: value_proj, sampling_offsets,
 * attention_weights and output_proj; DETR-to-Deformable-DETR article,
 * section 3.2), fp32 throughout, C = M * D channels:
 *
 *   value   = input_flatten W_v^T + b_v     [B, Nv, C], read as [B, Nv, M, D]
 *   offsets = query W_o^T + b_o             [B, Nq, M*L*K*2] = [B, Nq, M, L, K, 2]
 *   logits  = query W_a^T + b_a             [B, Nq, M*L*K]   = [B, Nq, M, L*K]
 *   core    = msda_forward_fused(value, reference_points, offsets, logits)
 *   output  = core W_out^T + b_out          [B, Nq, C]
 *
 * Weights are torch nn.Linear layouts: W_v, W_out [C, C]; W_o [M*L*K*2, C];
 * W_a [M*L*K, C]; biases [out features] or NULL for none. No padding mask
 * (every value row is a real pixel).
 */
typedef struct {
    const float *value_weight, *value_bias;    /* [C, C], [C]                   */
    const float *offset_weight, *offset_bias;  /* [M*L*K*2, C], [M*L*K*2]       */
    const float *attn_weight, *attn_bias;      /* [M*L*K, C], [M*L*K]           */
    const float *output_weight, *output_bias;  /* [C, C], [C]                   */
} msda_layer_params_t;

/* Gradients of the layer's parameters, same layouts; NULL skips one. */
typedef struct {
    float *value_weight, *value_bias;
    float *offset_weight, *offset_bias;
    float *attn_weight, *attn_bias;
    float *output_weight, *output_bias;
} msda_layer_grads_t;

/*
 * Forward of the layer. query [B, Nq, C], input_flatten [B, Nv, C],
 * reference_points [B, Nq, L, 2], output [B, Nq, C] (overwritten).
 * saved: caller-owned device buffer of msda_layer_saved_size() bytes,
 * 256-byte aligned; the forward writes value, offsets, logits and core into
 * it, and msda_layer_backward reads them. dims->D in {8, 16, 32, 64},
 * M*L*K >= 1. Alignment: query, input_flatten, output 16-byte;
 * reference_points 8-byte; weights 4-byte.
 */
msda_status_t msda_layer_forward(const msda_dims_t *dims, const float *query,
                                 const float *input_flatten, const float *reference_points,
                                 const int64_t *spatial_shapes, const int64_t *level_start_index,
                                 const msda_layer_params_t *params, float *output, void *saved,
                                 size_t saved_bytes, hipStream_t stream);

/*
 * Backward of the layer for grad_output [B, Nq, C], from the buffer `saved`
 * that msda_layer_forward filled with the same inputs and parameters.
 * Writes (each may be NULL): grad_query [B, Nq, C], grad_input_flatten
 * [B, Nv, C], grad_reference_points [B, Nq, L, 2] and the parameter
 * gradients in *grads (grads may be NULL). workspace: device scratch of
 * msda_layer_workspace_size() bytes, 256-byte aligned, clobbered.
 */
msda_status_t msda_layer_backward(const msda_dims_t *dims, const float *query,
                                  const float *input_flatten, const float *reference_points,
                                  const int64_t *spatial_shapes, const int64_t *level_start_index,
                                  const msda_layer_params_t *params, const void *saved,
                                  size_t saved_bytes, const float *grad_output, float *grad_query,
                                  float *grad_input_flatten, float *grad_reference_points,
                                  const msda_layer_grads_t *grads, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Bytes of the forward's saved activations and of the backward's workspace.
 * No HIP call. */
msda_status_t msda_layer_saved_size(const msda_dims_t *dims, size_t *bytes);
msda_status_t msda_layer_workspace_size(const msda_dims_t *dims, size_t *bytes);

/*
 * Grouped single-level deformable aggregation (DCNv3; deformable-attention
 * tutorial (discosf.com), section 4.2): for every output pixel p0 = (ho, wo), group g
 * and kernel point k = ky * kernel_w + kx,
 *
 *   output[b, ho, wo, g, :] = sum_k mask[b, ho, wo, g, k] *
 *                             bilinear(input[b, :, :, g, :], p0 + p_k + offset[b, ho, wo, g, k])
 *
 * with the convolution grid  p0 + p_k = (wo * stride_w - pad_w + kx * dilation_w,
 *                                         ho * stride_h - pad_h + ky * dilation_h)
 * in input pixels (x along W, y along H; pixel (i, j) sits at x = j, y = i),
 * the offset (x, y) in pixels added in fp32, bilinear interpolation over the
 * four surrounding pixels with zero outside the input, and the modulation
 * scalars used as given (no normalization). It is the core on one level with
 * the groups as heads (the shared projection w_g is a separate linear layer).
 *
 *   input   [B, H, W, G, D]           fp32 or bf16 (channels-last, grouped)
 *   offset  [B, H_out, W_out, G, K, 2] fp32, K = kernel_h * kernel_w
 *   mask    [B, H_out, W_out, G, K]    fp32
 *   output  [B, H_out, W_out, G * D]   fp32
 * D in {8, 16, 32, 64}; coordinates of the grid below 2^24.
 */
typedef struct {
    int64_t B, H, W, G, D;
    int64_t kernel_h, kernel_w;
    int64_t stride_h, stride_w;
    int64_t pad_h, pad_w;
    int64_t dilation_h, dilation_w;
    int64_t H_out, W_out;
} msda_dcn_dims_t;

/* Forward. Alignment: input and output 16-byte, offset 8-byte, mask 4-byte. */
msda_status_t msda_dcn_forward(const msda_dcn_dims_t *dims, msda_dtype_t input_dtype,
                               const void *input, const float *offset, const float *mask,
                               float *output, hipStream_t stream);

/*
 * Backward for grad_output [B, H_out, W_out, G * D]:
 *   grad_input  [B, H, W, G, D] fp32   (scattered without atomics, as grad_value)
 *   grad_offset [B, H_out, W_out, G, K, 2] = mask * sum_d g * d sample / d (x, y)
 *   grad_mask   [B, H_out, W_out, G, K]    = sum_d g * sample
 * each overwritten, each may be NULL. workspace as msda_backward: at least
 * msda_dcn_backward_workspace_size() bytes, 256-byte aligned, when
 * grad_input is requested.
 */
msda_status_t msda_dcn_backward(const msda_dcn_dims_t *dims, msda_dtype_t input_dtype,
                                const void *input, const float *offset, const float *mask,
                                const float *grad_output, float *grad_input, float *grad_offset,
                                float *grad_mask, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Bytes of workspace msda_dcn_backward needs. No HIP call. */
msda_status_t msda_dcn_backward_workspace_size(const msda_dcn_dims_t *dims,
                                               msda_dtype_t input_dtype, size_t *bytes);

/* Host-side check of a HOST copy of the level tables against Nv: every
 * H_l, W_l >= 1, level_start_index the prefix sums, sum H_l*W_l == Nv.
 * Returns MSDA_SUCCESS or MSDA_ERROR_INVALID_VALUE. No HIP call. */
msda_status_t msda_check_tables(const int64_t *host_spatial_shapes,
                                const int64_t *host_level_start_index, int64_t L, int64_t Nv);

/* Static description of a status code (never NULL). */
const char *msda_status_string(msda_status_t status);

/* MAJOR*10000 + MINOR*100 + PATCH. */
int msda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H_ */
