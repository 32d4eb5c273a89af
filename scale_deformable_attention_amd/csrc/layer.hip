// layer.hip -- the whole MSDeformAttn layer: the four projections around the
// fused core (deformable-attention tutorial (discosf.com), section 3.1: value_proj,
// sampling_offsets, attention_weights and output_proj linear layers;
// DETR-to-Deformable-DETR article, section 3.2: offsets viewed per head,
// level and point, the weights' softmax over L*K, offset / (W, H) added to the
// reference points). Host orchestration only: every step is a kernel of
// linear.hip (matrix cores) or msda.hip (the fused core), all on the caller's
// stream.
//
//   value   = input_flatten W_v^T + b_v        [B, Nv, C] = [B, Nv, M, D]
//   offsets = query W_o^T + b_o                [B, Nq, M*L*K*2] = [B, Nq, M, L, K, 2]
//   logits  = query W_a^T + b_a                [B, Nq, M*L*K]   = [B, Nq, M, L*K]
//   core    = fused core                       [B, Nq, C]
//   output  = core W_out^T + b_out             [B, Nq, C]
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gemm.h"
#include "msda.h"

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct LayerSizes {
    int64_t C, P, A;         // channels, offset features (M*L*K*2), logit features (M*L*K)
    int64_t rows_q, rows_v;  // B*Nq, B*Nv
};

LayerSizes layer_sizes(const msda_dims_t* d) {
    LayerSizes s;
    s.C = d->M * d->D;
    s.A = d->M * d->L * d->K;
    s.P = 2 * s.A;
    s.rows_q = d->B * d->Nq;
    s.rows_v = d->B * d->Nv;
    return s;
}

// Activations a forward keeps for its backward, in the caller's buffer.
struct SavedPlan {
    size_t value = 0, offsets = 0, logits = 0, core = 0, bytes = 0;
};

SavedPlan saved_plan(const msda_dims_t* d) {
    const LayerSizes s = layer_sizes(d);
    SavedPlan p;
    size_t at = 0;
    p.value = at;
    at += up((size_t)s.rows_v * s.C * 4);
    p.offsets = at;
    at += up((size_t)s.rows_q * s.P * 4);
    p.logits = at;
    at += up((size_t)s.rows_q * s.A * 4);
    p.core = at;
    at += up((size_t)s.rows_q * s.C * 4);
    p.bytes = at;
    return p;
}

// Work items one matrix-core launch should offer: the resident 128 x 128
// blocks of the whole GPU.
constexpr int64_t kGemmSlots = kGemmResidentBlocks;

int64_t tiles_of(int64_t rows, int64_t cols) { return ((rows + 127) / 128) * ((cols + 127) / 128); }

// Reduction splits of the batched weight gradients of the offset, logit and
// value heads (one launch): about one round of work items for all three.
int batch_splits(const msda_dims_t* d) {
    const int64_t C = d->M * d->D, A = d->M * d->L * d->K, P = 2 * A;
    const int64_t tiles = tiles_of(P, C) + tiles_of(A, C) + tiles_of(C, C);
    const int64_t rows = std::max<int64_t>(1, std::min(d->B * d->Nq, d->B * d->Nv));
    int64_t s = kGemmSlots / tiles;
    s = std::min<int64_t>(s, (rows + 15) / 16);
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, 256));
}

// Backward scratch: the core's input and value gradients, the offset and
// logit gradients, the fused backward's workspace and the linear layers'
// split partials (the output head's first, then the three batched heads',
// each in its own region).
struct WsPlan {
    size_t dcore = 0, dvalue = 0, doff = 0, dlogits = 0, core_ws = 0, core_ws_bytes = 0,
           partials = 0, bytes = 0;
};

msda_status_t ws_plan(const msda_dims_t* d, WsPlan& p) {
    const LayerSizes s = layer_sizes(d);
    size_t core_ws = 0;
    const msda_status_t st = msda_backward_fused_workspace_size(d, MSDA_DTYPE_F32, &core_ws);
    if (st != MSDA_SUCCESS) return st;
    size_t at = 0;
    p.dcore = at;
    at += up((size_t)s.rows_q * s.C * 4);
    p.dvalue = at;
    at += up((size_t)s.rows_v * s.C * 4);
    p.doff = at;
    at += up((size_t)s.rows_q * s.P * 4);
    p.dlogits = at;
    at += up((size_t)s.rows_q * s.A * 4);
    p.core_ws = at;
    p.core_ws_bytes = core_ws;
    at += up(core_ws);
    p.partials = at;
    const size_t sb = (size_t)batch_splits(d);
    const size_t batched = sb * ((size_t)s.P * s.C + s.P + (size_t)s.A * s.C + s.A +
                                 (size_t)s.C * s.C + s.C);
    const size_t part = std::max(msda_linear_workspace_floats(s.rows_q, s.C, s.C), batched);
    at += up(part * 4);
    p.bytes = at;
    return MSDA_SUCCESS;
}

msda_status_t check_layer(const msda_dims_t* d) {
    if (!d) return MSDA_ERROR_INVALID_VALUE;
    size_t unused = 0;
    const msda_status_t st = msda_backward_fused_workspace_size(d, MSDA_DTYPE_F32, &unused);
    if (st != MSDA_SUCCESS) return st;
    const LayerSizes s = layer_sizes(d);
    // 32-bit GEMM sizes
    if (s.rows_q >= ((int64_t)1 << 30) || s.rows_v >= ((int64_t)1 << 30) || s.P >= (1 << 20))
        return MSDA_ERROR_NOT_SUPPORTED;
    if (s.A == 0) return MSDA_ERROR_NOT_SUPPORTED;   // a layer has sampling points
    return MSDA_SUCCESS;
}

bool params_ok(const msda_layer_params_t* w) {
    return w && w->value_weight && w->offset_weight && w->attn_weight && w->output_weight &&
           aligned_to(w->value_weight, 4) && aligned_to(w->offset_weight, 4) &&
           aligned_to(w->attn_weight, 4) && aligned_to(w->output_weight, 4) &&
           aligned_to(w->value_bias, 4) && aligned_to(w->offset_bias, 4) &&
           aligned_to(w->attn_bias, 4) && aligned_to(w->output_bias, 4);
}

// Weight gradient dW[o, i] = sum_r dy[r, o] x[r, i] with the bias gradient
// (sum_r dy[r, o]) from the same pass; either may be null.
msda_status_t weight_and_bias(int O, int I, int R, const float* dy, const float* x, float* gw,
                              float* gb, int splits, float* part, float* part_b,
                              hipStream_t stream) {
    if (gw)
        return msda_gemm(false, false, O, I, R, dy, O, x, I, gw, I, nullptr, false,
                         R == 0 ? 1 : splits, part, stream, gb, part_b);
    if (gb) return msda_colsum(R, O, dy, O, gb, splits, part_b, false, stream);
    return MSDA_SUCCESS;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

msda_status_t msda_layer_saved_size(const msda_dims_t* dims, size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    const msda_status_t st = check_layer(dims);
    if (st != MSDA_SUCCESS) return st;
    *bytes = saved_plan(dims).bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_layer_workspace_size(const msda_dims_t* dims, size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    msda_status_t st = check_layer(dims);
    if (st != MSDA_SUCCESS) return st;
    WsPlan p;
    st = ws_plan(dims, p);
    if (st != MSDA_SUCCESS) return st;
    *bytes = p.bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_layer_forward(const msda_dims_t* dims, const float* query,
                                 const float* input_flatten, const float* reference_points,
                                 const int64_t* spatial_shapes, const int64_t* level_start_index,
                                 const msda_layer_params_t* params, float* output, void* saved,
                                 size_t saved_bytes, hipStream_t stream) {
    const msda_status_t st = check_layer(dims);
    if (st != MSDA_SUCCESS) return st;
    if (!params_ok(params) || !spatial_shapes || !level_start_index) return MSDA_ERROR_INVALID_VALUE;
    const LayerSizes s = layer_sizes(dims);
    if ((s.rows_q && (!query || !reference_points || !output)) || (s.rows_v && !input_flatten))
        return MSDA_ERROR_INVALID_VALUE;
    const SavedPlan sp = saved_plan(dims);
    if (!saved || !aligned_to(saved, kAlign) || saved_bytes < sp.bytes) return MSDA_ERROR_INVALID_VALUE;
    if (!aligned_to(query, 16) || !aligned_to(input_flatten, 16) || !aligned_to(output, 16) ||
        !aligned_to(reference_points, 8))
        return MSDA_ERROR_INVALID_VALUE;
    float* value = at<float>(saved, sp.value);
    float* off = at<float>(saved, sp.offsets);
    float* logits = at<float>(saved, sp.logits);
    float* core = at<float>(saved, sp.core);
    const int C = (int)s.C, P = (int)s.P, A = (int)s.A;
    const int Rq = (int)s.rows_q, Rv = (int)s.rows_v;
    const msda_layer_params_t& w = *params;
    msda_status_t r;
    // y[r, o] = sum_i x[r, i] W[o, i]: the three input projections in one launch
    GemmSpec in[3];
    in[0].M = Rv, in[0].N = C, in[0].K = C, in[0].A = input_flatten, in[0].lda = C;
    in[0].B = w.value_weight, in[0].ldb = C, in[0].C = value, in[0].ldc = C;
    in[0].bias = w.value_bias;
    in[1].M = Rq, in[1].N = P, in[1].K = C, in[1].A = query, in[1].lda = C;
    in[1].B = w.offset_weight, in[1].ldb = C, in[1].C = off, in[1].ldc = P;
    in[1].bias = w.offset_bias;
    in[2].M = Rq, in[2].N = A, in[2].K = C, in[2].A = query, in[2].lda = C;
    in[2].B = w.attn_weight, in[2].ldb = C, in[2].C = logits, in[2].ldc = A;
    in[2].bias = w.attn_bias;
    r = msda_gemm_batch(in, 3, stream);
    if (r != MSDA_SUCCESS) return r;
    r = msda_forward_fused(dims, MSDA_DTYPE_F32, value, spatial_shapes, level_start_index,
                           reference_points, off, logits, core, stream);
    if (r != MSDA_SUCCESS) return r;
    return msda_gemm(true, true, Rq, C, C, core, C, w.output_weight, C, output, C, w.output_bias,
                     false, 1, nullptr, stream);
}

msda_status_t msda_layer_backward(const msda_dims_t* dims, const float* query,
                                  const float* input_flatten, const float* reference_points,
                                  const int64_t* spatial_shapes, const int64_t* level_start_index,
                                  const msda_layer_params_t* params, const void* saved,
                                  size_t saved_bytes, const float* grad_output, float* grad_query,
                                  float* grad_input_flatten, float* grad_reference_points,
                                  const msda_layer_grads_t* grads, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    msda_status_t st = check_layer(dims);
    if (st != MSDA_SUCCESS) return st;
    if (!params_ok(params) || !spatial_shapes || !level_start_index) return MSDA_ERROR_INVALID_VALUE;
    const LayerSizes s = layer_sizes(dims);
    if ((s.rows_q && (!query || !reference_points || !grad_output)) || (s.rows_v && !input_flatten))
        return MSDA_ERROR_INVALID_VALUE;
    const SavedPlan sp = saved_plan(dims);
    if (!saved || !aligned_to(saved, kAlign) || saved_bytes < sp.bytes) return MSDA_ERROR_INVALID_VALUE;
    WsPlan wp;
    st = ws_plan(dims, wp);
    if (st != MSDA_SUCCESS) return st;
    if (!workspace || !aligned_to(workspace, kAlign) || workspace_bytes < wp.bytes)
        return MSDA_ERROR_INVALID_VALUE;
    const msda_layer_grads_t none = {};
    const msda_layer_grads_t& g = grads ? *grads : none;
    const float* gw_all[] = {g.value_weight, g.value_bias, g.offset_weight, g.offset_bias,
                             g.attn_weight, g.attn_bias, g.output_weight, g.output_bias};
    for (const float* p : gw_all)
        if (!aligned_to(p, 4)) return MSDA_ERROR_INVALID_VALUE;
    if (!aligned_to(query, 16) || !aligned_to(input_flatten, 16) || !aligned_to(grad_output, 16) ||
        !aligned_to(grad_query, 16) || !aligned_to(grad_input_flatten, 16) ||
        !aligned_to(reference_points, 8) || !aligned_to(grad_reference_points, 8))
        return MSDA_ERROR_INVALID_VALUE;

    const msda_layer_params_t& w = *params;
    const float* value = at<const float>(const_cast<void*>(saved), sp.value);
    const float* off = at<const float>(const_cast<void*>(saved), sp.offsets);
    const float* logits = at<const float>(const_cast<void*>(saved), sp.logits);
    const float* core = at<const float>(const_cast<void*>(saved), sp.core);
    float* dcore = at<float>(workspace, wp.dcore);
    float* dvalue = at<float>(workspace, wp.dvalue);
    float* doff = at<float>(workspace, wp.doff);
    float* dlogits = at<float>(workspace, wp.dlogits);
    void* core_ws = at<void>(workspace, wp.core_ws);
    float* part = at<float>(workspace, wp.partials);
    const int C = (int)s.C, P = (int)s.P, A = (int)s.A;
    const int Rq = (int)s.rows_q, Rv = (int)s.rows_v;
    const int sq = msda_linear_splits(Rq, C, C);
    msda_status_t r;

    // output projection: dcore = dy W_out; dW_out = dy^T core; db_out = sum dy
    r = msda_gemm(true, false, Rq, C, C, grad_output, C, w.output_weight, C, dcore, C, nullptr,
                  false, 1, nullptr, stream);
    if (r != MSDA_SUCCESS) return r;
    r = weight_and_bias(C, C, Rq, grad_output, core, g.output_weight, g.output_bias, sq, part,
                        part + (size_t)sq * C * C, stream);
    if (r != MSDA_SUCCESS) return r;

    // the fused core: value, reference-point, offset and logit gradients
    const bool want_value = grad_input_flatten || g.value_weight || g.value_bias;
    const bool want_q = grad_query || g.offset_weight || g.offset_bias || g.attn_weight ||
                        g.attn_bias;
    r = msda_backward_fused(dims, MSDA_DTYPE_F32, value, spatial_shapes, level_start_index,
                            reference_points, off, logits, dcore, want_value ? dvalue : nullptr,
                            grad_reference_points, want_q ? doff : nullptr,
                            want_q ? dlogits : nullptr, core_ws, wp.core_ws_bytes, stream);
    if (r != MSDA_SUCCESS) return r;

    // input gradients in one launch: dquery = doff W_o + dlogits W_a (two
    // reduction segments of one product), dinput = dvalue W_v
    GemmSpec nn[2];
    int nnn = 0;
    if (grad_query && Rq > 0) {
        GemmSpec& q = nn[nnn++];
        q.a_kmajor = true, q.b_kmajor = false;
        q.M = Rq, q.N = C, q.K = P, q.A = doff, q.lda = P, q.B = w.offset_weight, q.ldb = C;
        q.C = grad_query, q.ldc = C;
        if (P % 16 == 0) {
            q.A2 = dlogits, q.lda2 = A, q.B2 = w.attn_weight, q.ldb2 = C, q.K2 = A;
        }
    }
    if (grad_input_flatten && Rv > 0) {
        GemmSpec& v = nn[nnn++];
        v.a_kmajor = true, v.b_kmajor = false;
        v.M = Rv, v.N = C, v.K = C, v.A = dvalue, v.lda = C, v.B = w.value_weight, v.ldb = C;
        v.C = grad_input_flatten, v.ldc = C;
    }
    if (nnn > 0) {
        r = msda_gemm_batch(nn, nnn, stream);
        if (r != MSDA_SUCCESS) return r;
    }
    if (grad_query && Rq > 0 && P % 16 != 0) {
        r = msda_gemm(true, false, Rq, C, A, dlogits, A, w.attn_weight, C, grad_query, C, nullptr,
                      true, 1, nullptr, stream);
        if (r != MSDA_SUCCESS) return r;
    }

    // weight (and bias) gradients of the offset, logit and value heads in one
    // launch, each product with its own partial buffers
    const int sb = batch_splits(dims);
    float* part_off = part;
    float* part_off_b = part_off + (size_t)sb * P * C;
    float* part_att = part_off_b + (size_t)sb * P;
    float* part_att_b = part_att + (size_t)sb * A * C;
    float* part_val = part_att_b + (size_t)sb * A;
    float* part_val_b = part_val + (size_t)sb * C * C;
    GemmSpec tn[3];
    int ntn = 0;
    struct Head {
        float *gw, *gb;
        int O, R;
        const float *dy, *x;
        float *part, *part_b;
    } heads[3] = {{g.offset_weight, g.offset_bias, P, Rq, doff, query, part_off, part_off_b},
                  {g.attn_weight, g.attn_bias, A, Rq, dlogits, query, part_att, part_att_b},
                  {g.value_weight, g.value_bias, C, Rv, dvalue, input_flatten, part_val,
                   part_val_b}};
    for (const Head& h : heads) {
        if (h.gw) {
            GemmSpec& t = tn[ntn++];
            t.a_kmajor = false, t.b_kmajor = false;
            t.M = h.O, t.N = C, t.K = h.R, t.A = h.dy, t.lda = h.O, t.B = h.x, t.ldb = C;
            t.C = h.gw, t.ldc = C, t.splits = h.R == 0 ? 1 : sb, t.partials = h.part;
            t.a_colsum = h.gb, t.a_colsum_partials = h.part_b;
        } else if (h.gb) {
            r = msda_colsum(h.R, h.O, h.dy, h.O, h.gb, sb, h.part_b, false, stream);
            if (r != MSDA_SUCCESS) return r;
        }
    }
    if (ntn > 0) return msda_gemm_batch(tn, ntn, stream);
    return MSDA_SUCCESS;
}

}  // extern "C"
