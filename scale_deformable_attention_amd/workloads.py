"""Seeded synthetic inputs for the multi-scale deformable attention core.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds none of the core's arithmetic (no coordinate map, no
interpolation, no weighted sum): it only draws random numbers with numpy and
assembles the six tensors the core takes.

Two model-side steps that sit *before* the core are used to shape realistic
inputs, both as the DETR-to-Deformable-DETR article (cf-1.com, section 3.2)
describes them:
  * sampling locations = reference point + offset / (W_l, H_l), with raw
    offsets drawn in level-l pixels;
  * attention weights = softmax of logits over the L*K samples of one
    (query, head) (also the CSDN MSDA explainer, section 3, note 3).

Reference points: encoder queries are the pixel centres of every level,
normalized to [0, 1] (cf-1.com section 3.2: position plus half a pixel); the
decoder and the tiny case draw them uniformly.

Shapes are those of the 800x1333 and 1920x1080 feature pyramids at strides
8/16/32/64 with the Deformable-DETR defaults M=8 heads, L=4 levels, K=4
points, d_model 256 (discosf.com section 2.2; cf-1.com section 3.3). Values,
offsets, logits and upstream gradients are normal draws; they stand in for
real activations (no dataset is used).

Draw order per workload (numpy PCG64, seed fixed per workload): value,
reference points (when random), offsets, logits, upstream gradient.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

PYRAMID_800x1333 = ((100, 167), (50, 84), (25, 42), (13, 21))
PYRAMID_1920x1080 = ((135, 240), (68, 120), (34, 60), (17, 30))


@dataclass(frozen=True)
class Workload:
    """One synthetic workload of the core.

    ref: "grid" (every pixel of every level is a query, Nq = Nv),
         "uniform" (U[0,1]^2) or "inner" (U[0.05,0.95]^2).
    sigma_px: standard deviation of the sampling offsets, in level-l pixels.
    """
    name: str
    B: int
    M: int
    D: int
    K: int
    shapes: Tuple[Tuple[int, int], ...]
    ref: str
    sigma_px: float
    Nq: Optional[int] = None
    value_dtype: str = "f32"
    backward: bool = False
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def L(self):
        return len(self.shapes)

    @property
    def Nv(self):
        return int(sum(h * w for h, w in self.shapes))

    @property
    def num_queries(self):
        return self.Nv if self.ref == "grid" else int(self.Nq)

    @property
    def points(self):
        """Sampled points per pass, B*Nq*M*L*K (the metric's unit)."""
        return self.B * self.num_queries * self.M * self.L * self.K

    def level_start_index(self):
        starts, s = [], 0
        for h, w in self.shapes:
            starts.append(s)
            s += h * w
        return np.asarray(starts, np.int64)

    def scaled(self, **changes):
        """A copy with some fields changed (used to make small test cases)."""
        d = {k: getattr(self, k) for k in self.__dataclass_fields__}
        d.update(changes)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, M=2, D=8, K=2, shapes=((8, 8), (4, 4)), ref="uniform",
                     sigma_px=1.0, Nq=16, backward=True, seed=1001,
                     note="tiny fp32 fwd+bwd"),
    "encoder": Workload("encoder", B=2, M=8, D=32, K=4, shapes=PYRAMID_800x1333, ref="grid",
                        sigma_px=2.0, seed=1002,
                        note="800x1333 encoder self-attention, fp32, forward"),
    "decoder": Workload("decoder", B=8, M=8, D=32, K=4, shapes=PYRAMID_800x1333, ref="inner",
                        sigma_px=4.0, Nq=300, backward=True, seed=1003,
                        note="800x1333 decoder cross-attention, 300 queries, fp32 fwd+bwd"),
    "hires_bf16": Workload("hires_bf16", B=2, M=8, D=32, K=8, shapes=PYRAMID_1920x1080,
                           ref="grid", sigma_px=3.0, value_dtype="bf16", seed=1004,
                           note="1920x1080 encoder, bf16 value, fp32 accumulate, forward"),
    "encoder_train": Workload("encoder_train", B=4, M=8, D=32, K=4, shapes=PYRAMID_800x1333,
                              ref="grid", sigma_px=8.0, backward=True, seed=1005,
                              note="800x1333 encoder training step, fp32 fwd+bwd"),
}


def bf16_round(x):
    """Round float32 to the nearest bfloat16 (ties to even). Returns the bf16
    bit patterns as uint16. NaN stays NaN (quiet)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, np.float32))
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _reference_points(w, rng):
    """Normalized reference point of every query, [Nq, 2] as (x, y)."""
    if w.ref == "grid":
        refs = []
        for h, wd in w.shapes:
            jj, ii = np.meshgrid((np.arange(wd) + 0.5) / wd, (np.arange(h) + 0.5) / h)
            refs.append(np.stack([jj.reshape(-1), ii.reshape(-1)], -1))
        return np.concatenate(refs, 0)
    lo, hi = (0.0, 1.0) if w.ref == "uniform" else (0.05, 0.95)
    return rng.uniform(lo, hi, size=(w.Nq, 2))


def generate(w: Workload, batch_slice=None):
    """Draw the inputs of one workload.

    Returns a dict of numpy arrays:
      value            [B,Nv,M,D] float32 (for bf16 workloads: the bf16-rounded
                       values widened to float32, exactly what the GPU reads)
      value_bf16       [B,Nv,M,D] uint16 bf16 bits (bf16 workloads only)
      value_f16        [B,Nv,M,D] float16 (f16 workloads only)
      value_f32_orig   the unrounded float32 draws (bf16 and f16 workloads)
      spatial_shapes   [L,2] int64 (H, W)
      level_start_index[L] int64
      sampling_locations [B,Nq,M,L,K,2] float32
      attention_weights  [B,Nq,M,L,K] float32
      grad_output      [B,Nq,M*D] float32
      reference_points [Nq,2] float64 (x, y) normalized
    and the raw draws, as the fused front-end takes them:
      reference_points_levels [B,Nq,L,2] float32 (the query's point, the same
                       on every level)
      sampling_offsets   [B,Nq,M,L,K,2] float32, level pixels
      attention_logits   [B,Nq,M,L*K] float32
    ``batch_slice`` (a slice over B) keeps only those batch entries; the draws
    are made for the full batch first so a slice is a true sub-sample.
    """
    rng = np.random.default_rng(w.seed)
    B, M, D, L, K, Nv, Nq = w.B, w.M, w.D, w.L, w.K, w.Nv, w.num_queries
    value = rng.standard_normal((B, Nv, M, D), dtype=np.float32)
    ref = _reference_points(w, rng)                                   # [Nq, 2]
    offsets = rng.standard_normal((B, Nq, M, L, K, 2)) * w.sigma_px    # level pixels
    logits = rng.standard_normal((B, Nq, M, L * K))
    grad_output = rng.standard_normal((B, Nq, M * D), dtype=np.float32)

    wh = np.asarray([[wd, h] for h, wd in w.shapes], np.float64)       # [L, 2] as (W, H)
    loc = ref[None, :, None, None, None, :] + offsets / wh[None, None, None, :, None, :]
    e = np.exp(logits - logits.max(-1, keepdims=True))
    attn = (e / e.sum(-1, keepdims=True)).reshape(B, Nq, M, L, K)

    out = {
        "spatial_shapes": np.asarray(w.shapes, np.int64).reshape(L, 2),
        "level_start_index": w.level_start_index(),
        "sampling_locations": loc.astype(np.float32),
        "attention_weights": attn.astype(np.float32),
        "grad_output": grad_output,
        "reference_points": ref,
        "reference_points_levels": np.ascontiguousarray(np.broadcast_to(
            ref.astype(np.float32)[None, :, None, :], (B, Nq, L, 2))),
        "sampling_offsets": offsets.astype(np.float32),
        "attention_logits": logits.astype(np.float32),
    }
    if w.value_dtype == "bf16":
        bits = bf16_round(value)
        out["value_bf16"] = bits
        out["value_f32_orig"] = value
        out["value"] = bf16_to_f32(bits)
    elif w.value_dtype == "f16":
        half = value.astype(np.float16)          # round to nearest even
        out["value_f16"] = half
        out["value_f32_orig"] = value
        out["value"] = half.astype(np.float32)   # exact
    else:
        out["value"] = value
    if batch_slice is not None:
        for key in ("value", "value_bf16", "value_f16", "value_f32_orig", "sampling_locations",
                    "attention_weights", "grad_output", "reference_points_levels",
                    "sampling_offsets", "attention_logits"):
            if key in out:
                out[key] = np.ascontiguousarray(out[key][batch_slice])
    return out


def _dyadic(rng, shape, bound, step_log2):
    """Uniform draws on the grid k * 2^-step_log2 within [-bound, bound], as
    float32 (exactly representable)."""
    n = int(round(bound * 2.0 ** step_log2))
    return (rng.integers(-n, n + 1, size=shape).astype(np.float64) *
            2.0 ** -step_log2).astype(np.float32)


def generate_layer(w: Workload, offset_px=8.0):
    """Seeded inputs and parameters of the MSDeformAttn layer around the core
    at the workload's sizes (C = M * D channels).

    Every activation, weight, bias and upstream gradient is drawn uniformly on
    a dyadic grid (a stand-in for xavier-uniform weights and normalized
    activations): query and input_flatten in [-1, 1] with step 1/16, weights
    with step 2^-9 and biases with step 2^-9 or 1/16. With C <= 256 channels
    every product and partial sum of the offset, logit, value and
    upstream-gradient projections then stays on a grid of 2^-13 with magnitude
    below 2^10 (at most 23 significant bits), so those projections are exact in
    single precision whatever the summation order, and two correct
    implementations sample at exactly the same locations.

    Offset weights are scaled so that the offsets have a standard deviation of
    about ``offset_px`` level pixels; their bias follows the pages' start-up
    pattern rounded to 1/16 (head m points along angle 2 pi m / M, point k at
    k + 1 pixels; DETR-to-Deformable-DETR article, section 3.2).
    """
    rng = np.random.default_rng(w.seed + 7919)
    B, M, D, L, K, Nv, Nq = w.B, w.M, w.D, w.L, w.K, w.Nv, w.num_queries
    C = M * D
    if C > 256:
        raise ValueError("exactness of the projections is arranged for C <= 256")
    A = M * L * K
    x = {}
    x["query"] = _dyadic(rng, (B, Nq, C), 1.0, 4)
    x["input_flatten"] = _dyadic(rng, (B, Nv, C), 1.0, 4)
    # std of sum_i q_i w_i with q ~ U[-1,1], w ~ U[-a,a]: a * sqrt(C) / 3
    a_off = min(4.0, offset_px * 3.0 / np.sqrt(C))
    x["offset_weight"] = _dyadic(rng, (2 * A, C), a_off, 9)
    th = 2.0 * np.pi * np.arange(M) / M
    dirs = np.stack([np.cos(th), np.sin(th)], -1)
    dirs = dirs / np.abs(dirs).max(-1, keepdims=True)
    grid = np.repeat(dirs[:, None, None, :], L, 1).repeat(K, 2) * \
        (np.arange(K) + 1)[None, None, :, None]
    x["offset_bias"] = (np.round(grid.reshape(-1) * 16) / 16).astype(np.float32)
    x["attn_weight"] = _dyadic(rng, (A, C), 0.125, 9)
    x["attn_bias"] = _dyadic(rng, (A,), 0.25, 9)
    x["value_weight"] = _dyadic(rng, (C, C), 0.125, 9)
    x["value_bias"] = _dyadic(rng, (C,), 0.125, 9)
    x["output_weight"] = _dyadic(rng, (C, C), 0.125, 9)
    x["output_bias"] = _dyadic(rng, (C,), 0.125, 9)
    x["grad_output"] = _dyadic(rng, (B, Nq, C), 1.0, 4)
    ref = _reference_points(w, rng).astype(np.float32)
    x["reference_points"] = np.ascontiguousarray(
        np.broadcast_to(ref[None, :, None, :], (B, Nq, L, 2)))
    x["spatial_shapes"] = np.asarray(w.shapes, np.int64).reshape(L, 2)
    x["level_start_index"] = w.level_start_index()
    return x


@dataclass(frozen=True)
class DcnWorkload:
    """One synthetic workload of the grouped single-level aggregation (DCNv3):
    input [B, H, W, G, D], a kernel_h x kernel_w grid per output pixel."""
    name: str
    B: int
    H: int
    W: int
    G: int
    D: int
    kernel: Tuple[int, int] = (3, 3)
    stride: Tuple[int, int] = (1, 1)
    pad: Tuple[int, int] = (1, 1)
    dilation: Tuple[int, int] = (1, 1)
    sigma_px: float = 1.0
    value_dtype: str = "f32"
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def K(self):
        return self.kernel[0] * self.kernel[1]

    @property
    def out_size(self):
        return ((self.H + 2 * self.pad[0] - self.dilation[0] * (self.kernel[0] - 1) - 1)
                // self.stride[0] + 1,
                (self.W + 2 * self.pad[1] - self.dilation[1] * (self.kernel[1] - 1) - 1)
                // self.stride[1] + 1)

    @property
    def points(self):
        Ho, Wo = self.out_size
        return self.B * Ho * Wo * self.G * self.K


# InternImage-style stages on the 800x1333 detection input: 16 channels per
# group at every stage (64 channels in 4 groups at stride 4, 128 in 8 at
# stride 8), 3x3 grids (deformable-attention tutorial (discosf.com), sections 4.2 and
# 5.2: G between 4 and 16, G=8 with K=9 as the typical pairing).
DCN_WORKLOADS = {
    "dcn_tiny": DcnWorkload("dcn_tiny", B=1, H=6, W=7, G=2, D=8, sigma_px=1.0, seed=2001,
                            note="tiny 3x3 fp32 fwd+bwd"),
    "dcnv3_stage2": DcnWorkload("dcnv3_stage2", B=4, H=100, W=167, G=8, D=16, sigma_px=2.0,
                                seed=2002, note="stride-8 stage of the 800x1333 input, "
                                                "C=128 in 8 groups, 3x3, fp32 fwd+bwd"),
    "dcnv3_stage1": DcnWorkload("dcnv3_stage1", B=2, H=200, W=334, G=4, D=16, sigma_px=2.0,
                                seed=2003, note="stride-4 stage of the 800x1333 input, "
                                                "C=64 in 4 groups, 3x3, fp32 fwd+bwd"),
}


def generate_dcn(w: DcnWorkload):
    """Seeded inputs of a DCNv3 workload: input normal (bf16-rounded for bf16
    workloads), offsets normal with standard deviation sigma_px pixels,
    modulation scalars a softmax over the K grid points of normal logits (the
    normalization InternImage applies; the aggregation itself uses them as
    given), upstream gradient normal."""
    rng = np.random.default_rng(w.seed)
    Ho, Wo = w.out_size
    x = {}
    inp = rng.standard_normal((w.B, w.H, w.W, w.G, w.D), dtype=np.float32)
    off = (rng.standard_normal((w.B, Ho, Wo, w.G, w.K, 2)) * w.sigma_px).astype(np.float32)
    z = rng.standard_normal((w.B, Ho, Wo, w.G, w.K))
    e = np.exp(z - z.max(-1, keepdims=True))
    x["mask"] = (e / e.sum(-1, keepdims=True)).astype(np.float32)
    x["offset"] = off
    x["grad_output"] = rng.standard_normal((w.B, Ho, Wo, w.G * w.D), dtype=np.float32)
    if w.value_dtype == "bf16":
        bits = bf16_round(inp)
        x["input_bf16"] = bits
        x["input"] = bf16_to_f32(bits)
    elif w.value_dtype == "f16":
        half = inp.astype(np.float16)
        x["input_f16"] = half
        x["input"] = half.astype(np.float32)
    else:
        x["input"] = inp
    return x
