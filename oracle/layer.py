"""CPU oracle of the layer around the deformable attention core (test
infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product path never does).

The layer is MSDeformAttn as the pages build it (deformable-attention
tutorial (discosf.com), section 3.1, the module with sampling_offsets,
attention_weights, value_proj and output_proj linear layers;
DETR-to-Deformable-DETR article, section 3.2, the forward that views the
offsets as [B, Nq, M, L, K, 2], takes the softmax of the weights over L*K and
adds offset / (W, H) to the reference points):

    value   = input_flatten W_v^T + b_v                  viewed [B, Nv, M, D]
    offsets = query W_o^T + b_o                          viewed [B, Nq, M, L, K, 2]
    logits  = query W_a^T + b_a                          viewed [B, Nq, M, L*K]
    core    = fused core (reference points, offsets, softmax(logits))
    output  = core W_out^T + b_out

Linear layers are numpy double matmuls (a library primitive, no blocking or
reordering beyond the definition). The core is the C oracle's fused function,
fed the offsets and logits rounded to single precision: the layer's tensors
between steps are single-precision tensors, and the core's reading of the
location (single-precision quotient and sum) starts from them.

Every function can also return, for each result, S: the sum of the absolute
values of the terms that make it up, propagated through the steps (an
absolute-value pass: |x| |W|^T + |b| for a linear layer, the core evaluated on
the bound of its value input, the core's gradients on the bounds of value and
upstream gradient). The GPU parity tests bound their error by it.
"""
import numpy as np

from . import backward_fused, forward_fused


# ----------------------------------------------------------------------------- linear
def linear_forward(x, w, b=None, with_abs=False):
    """y = x W^T + b in double; x [..., I], w [O, I], b [O]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    y = x @ w.T
    if b is not None:
        y = y + np.asarray(b, np.float64)
    if not with_abs:
        return y
    s = np.abs(x) @ np.abs(w).T
    if b is not None:
        s = s + np.abs(np.asarray(b, np.float64))
    return y, s


def linear_backward(x, w, gy, with_abs=False):
    """(grad_x, grad_w, grad_b) of y = x W^T + b for the upstream gradient gy,
    in double: grad_x = gy W, grad_w = gy^T x, grad_b = sum of gy over rows."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    gy = np.asarray(gy, np.float64)
    I = w.shape[1]
    O = w.shape[0]
    x2 = x.reshape(-1, I)
    g2 = gy.reshape(-1, O)
    gx = (g2 @ w).reshape(x.shape)
    gw = g2.T @ x2
    gb = g2.sum(0)
    if not with_abs:
        return gx, gw, gb
    ax, aw, ag = np.abs(x2), np.abs(w), np.abs(g2)
    return gx, gw, gb, (ag @ aw).reshape(x.shape), ag.T @ ax, ag.sum(0)


def _abs_bound_linear(s_x, w, b=None):
    """Propagated bound: S_y = S_x |W|^T (+ |b|)."""
    s = s_x @ np.abs(np.asarray(w, np.float64)).T
    if b is not None:
        s = s + np.abs(np.asarray(b, np.float64))
    return s


# ----------------------------------------------------------------------------- layer
def _views(B, Nq, M, L, K):
    return (B, Nq, M, L, K, 2), (B, Nq, M, L * K)


def layer_forward(p, query, input_flatten, reference_points, spatial_shapes,
                  level_start_index, M, L, K, with_abs=False, keep=False):
    """MSDeformAttn forward. p: dict of weights w_value [C, C], b_value [C],
    w_offset [M*L*K*2, C], b_offset, w_attn [M*L*K, C], b_attn, w_out [C, C],
    b_out. query [B, Nq, C], input_flatten [B, Nv, C], reference_points
    [B, Nq, L, 2]. Returns output [B, Nq, C] (and its S with ``with_abs``;
    the intermediate tensors too with ``keep``)."""
    query = np.asarray(query, np.float64)
    inp = np.asarray(input_flatten, np.float64)
    B, Nq, C = query.shape
    Nv = inp.shape[1]
    D = C // M
    so, sl = _views(B, Nq, M, L, K)
    value = linear_forward(inp, p["w_value"], p["b_value"])
    off = linear_forward(query, p["w_offset"], p["b_offset"]).astype(np.float32).reshape(so)
    logits = linear_forward(query, p["w_attn"], p["b_attn"]).astype(np.float32).reshape(sl)
    v4 = value.reshape(B, Nv, M, D)
    core = forward_fused(v4, spatial_shapes, level_start_index, reference_points, off, logits)
    core = core.reshape(B, Nq, C)
    out = linear_forward(core, p["w_out"], p["b_out"])
    res = [out]
    if with_abs:
        s_value = _abs_bound_linear(np.abs(inp), p["w_value"], p["b_value"]).reshape(B, Nv, M, D)
        # the core's terms A * w_c * v with |v| bounded by S_value (A, w_c >= 0)
        s_core = forward_fused(s_value, spatial_shapes, level_start_index, reference_points,
                               off, logits).reshape(B, Nq, C)
        res.append(_abs_bound_linear(s_core, p["w_out"], p["b_out"]))
    if keep:
        res.append(dict(value=v4, offsets=off, logits=logits, core=core))
    return tuple(res) if len(res) > 1 else out


def layer_backward(p, query, input_flatten, reference_points, spatial_shapes,
                   level_start_index, M, L, K, grad_output, with_abs=False):
    """Gradients of layer_forward for grad_output [B, Nq, C]: a dict with
    query, input_flatten, reference_points and every weight and bias
    (w_value, b_value, ...). With ``with_abs`` also a dict of their S."""
    query = np.asarray(query, np.float64)
    inp = np.asarray(input_flatten, np.float64)
    gy = np.asarray(grad_output, np.float64)
    B, Nq, C = query.shape
    Nv = inp.shape[1]
    D = C // M
    _, keep = layer_forward(p, query, inp, reference_points, spatial_shapes, level_start_index,
                            M, L, K, keep=True)
    value, off, logits, core = keep["value"], keep["offsets"], keep["logits"], keep["core"]
    g = {}
    dcore, g["w_out"], g["b_out"] = linear_backward(core, p["w_out"], gy)
    gv, gref, goff, glog = backward_fused(value, spatial_shapes, level_start_index,
                                          reference_points, off, logits, dcore.reshape(B, Nq, C))
    g["reference_points"] = gref
    goff2 = goff.reshape(B, Nq, -1)
    glog2 = glog.reshape(B, Nq, -1)
    gq1, g["w_offset"], g["b_offset"] = linear_backward(query, p["w_offset"], goff2)
    gq2, g["w_attn"], g["b_attn"] = linear_backward(query, p["w_attn"], glog2)
    g["query"] = gq1 + gq2
    g["input_flatten"], g["w_value"], g["b_value"] = linear_backward(
        inp, p["w_value"], gv.reshape(B, Nv, C))
    if not with_abs:
        return g
    s = {}
    ag = np.abs(gy).reshape(-1, C)
    aw_out = np.abs(np.asarray(p["w_out"], np.float64))
    s_dcore = (ag @ aw_out).reshape(B, Nq, C)
    s_value = _abs_bound_linear(np.abs(inp), p["w_value"], p["b_value"]).reshape(B, Nv, M, D)
    s_core = forward_fused(s_value, spatial_shapes, level_start_index, reference_points, off,
                           logits).reshape(-1, C)
    s["w_out"] = ag.T @ s_core
    s["b_out"] = ag.sum(0)
    # the core's gradient terms with |value| <= S_value and |upstream| <= S_dcore
    res = backward_fused(s_value, spatial_shapes, level_start_index, reference_points, off,
                         logits, s_dcore, with_abs=True)
    s_gv, s_gref, s_goff, s_glog = res[4:]
    s["reference_points"] = s_gref
    s_goff2 = s_goff.reshape(-1, M * L * K * 2)
    s_glog2 = s_glog.reshape(-1, M * L * K)
    aq = np.abs(query).reshape(-1, C)
    s["query"] = (s_goff2 @ np.abs(np.asarray(p["w_offset"], np.float64)) +
                  s_glog2 @ np.abs(np.asarray(p["w_attn"], np.float64))).reshape(B, Nq, C)
    s["w_offset"] = s_goff2.T @ aq
    s["b_offset"] = s_goff2.sum(0)
    s["w_attn"] = s_glog2.T @ aq
    s["b_attn"] = s_glog2.sum(0)
    s_gv2 = s_gv.reshape(-1, C)
    s["input_flatten"] = (s_gv2 @ np.abs(np.asarray(p["w_value"], np.float64))).reshape(B, Nv, C)
    s["w_value"] = s_gv2.T @ np.abs(inp).reshape(-1, C)
    s["b_value"] = s_gv2.sum(0)
    return g, s
