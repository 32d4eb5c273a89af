"""GPU parity of the reduced-precision storage variants against the CPU
oracle, through the C ABI:

* value stored as IEEE binary16 (core, fused front-end, DCNv3);
* sampling locations and attention weights stored as binary16;
* grad_value written as bf16.

Narrow inputs are widened exactly by the kernels, so the oracle is fed the
same narrow values widened to float and the fp32 tolerance applies
(|x - r| <= 1e-5 |r| + 1e-5 S). A bf16 grad_value is the fp32 result rounded
to nearest even: half a bf16 unit, 2^-9 relative, on top of the fp32 bound,
so that output is held to |x - r| <= 2^-8 |r| + 1e-5 S.
"""
import numpy as np
import pytest

import oracle
from scale_deformable_attention_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

STOL = 1e-5
RTOL = 1e-5
RTOL_BF16_OUT = 2.0 ** -8
SMALL_PYRAMID = ((13, 21), (7, 11), (4, 6), (2, 3))


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scale_deformable_attention_amd as msda
    msda.library()
    return torch.device("cuda:0")


def check(name, got, ref, ref_abs, rtol):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= rtol * np.abs(ref) + STOL * ref_abs)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{i.tolist()}: gpu {got.reshape(-1)[i]} oracle {ref.reshape(-1)[i]} "
                             f"abs-sum {ref_abs.reshape(-1)[i]}")
    denom = np.abs(ref) + ref_abs
    big = denom > 0
    rel = float(np.max(err[big] / denom[big])) if big.any() else 0.0
    print(f"  {name}: max |gpu-oracle| / (|r| + S) = {rel:.2e}", flush=True)


def bf16_tensor_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def core_case(w, half_locations, value_dtype, grad_bf16, x=None):
    """Run the core through the binding with the given storage precisions and
    compare with the oracle fed the same narrow values."""
    dev = _dev()
    import scale_deformable_attention_amd as msda
    print(f"[precision] {w.name}: value {value_dtype}, locations "
          f"{'f16' if half_locations else 'f32'}, grad_value {'bf16' if grad_bf16 else 'f32'}",
          flush=True)
    x = x if x is not None else wl.generate(w)
    if value_dtype == "f16":
        value = torch.from_numpy(x["value_f16"]).to(dev)
    elif value_dtype == "bf16":
        value = torch.from_numpy(x["value_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        value = torch.from_numpy(x["value"]).to(dev)
    loc, attn = x["sampling_locations"], x["attention_weights"]
    if half_locations:
        loc, attn = loc.astype(np.float16), attn.astype(np.float16)
    T = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
         for k, v in (("shapes", x["spatial_shapes"]), ("lsi", x["level_start_index"]),
                      ("loc", loc), ("attn", attn), ("g", x["grad_output"]))}
    out = msda.msda_forward(value, T["shapes"], T["lsi"], T["loc"], T["attn"])
    gv, gl, ga = msda.msda_backward(value, T["shapes"], T["lsi"], T["loc"], T["attn"], T["g"],
                                    grad_value_dtype=torch.bfloat16 if grad_bf16
                                    else torch.float32)
    torch.cuda.synchronize()
    assert gv.dtype == (torch.bfloat16 if grad_bf16 else torch.float32)
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], loc.astype(np.float32),
            attn.astype(np.float32))
    ref, ref_abs = oracle.forward(*args, with_abs=True)
    check("output", out.cpu().numpy(), ref, ref_abs, RTOL)
    rgv, rgl, rga, agv, agl, aga = oracle.backward(*args, x["grad_output"], with_abs=True)
    check("grad_value", bf16_tensor_to_f64(gv), rgv, agv, RTOL_BF16_OUT if grad_bf16 else RTOL)
    check("grad_sampling_locations", gl.cpu().numpy(), rgl, agl, RTOL)
    check("grad_attention_weights", ga.cpu().numpy(), rga, aga, RTOL)


@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_f16_value_every_head_width(D):
    w = wl.Workload(f"f16_D{D}", B=2, M=5, D=D, K=3, shapes=SMALL_PYRAMID[:3], ref="uniform",
                    sigma_px=2.0, Nq=37, value_dtype="f16", seed=500 + D)
    core_case(w, half_locations=False, value_dtype="f16", grad_bf16=False)


@pytest.mark.parametrize("D", [8, 32])
def test_half_locations_and_weights(D):
    w = wl.Workload(f"hloc_D{D}", B=2, M=4, D=D, K=4, shapes=SMALL_PYRAMID, ref="uniform",
                    sigma_px=3.0, Nq=41, seed=510 + D)
    core_case(w, half_locations=True, value_dtype="f32", grad_bf16=False)


def test_half_locations_with_staged_levels():
    w = wl.Workload("hloc_staged", B=1, M=2, D=32, K=4,
                    shapes=((64, 96), (32, 48), (16, 24), (8, 12)), ref="uniform",
                    sigma_px=3.0, Nq=2500, seed=530)
    core_case(w, half_locations=True, value_dtype="f32", grad_bf16=False)


@pytest.mark.parametrize("D", [32, 64])
def test_f16_values_with_staged_levels(D):
    # 64- and 128-byte binary16 rows: the forward stages the coarse levels
    w = wl.Workload(f"f16_staged_D{D}", B=1, M=4, D=D, K=4,
                    shapes=((64, 96), (32, 48), (16, 24), (8, 12)), ref="uniform",
                    sigma_px=3.0, Nq=2300, value_dtype="f16", seed=531 + D)
    core_case(w, half_locations=False, value_dtype="f16", grad_bf16=False)


@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_bf16_grad_value(D):
    w = wl.Workload(f"bf16out_D{D}", B=2, M=4, D=D, K=3, shapes=SMALL_PYRAMID[:3],
                    ref="uniform", sigma_px=2.0, Nq=29, seed=520 + D)
    core_case(w, half_locations=False, value_dtype="f32", grad_bf16=True)


def test_all_narrow_together():
    w = wl.Workload("narrow_all", B=2, M=8, D=32, K=4, shapes=SMALL_PYRAMID, ref="grid",
                    sigma_px=3.0, value_dtype="bf16", seed=530)
    core_case(w, half_locations=True, value_dtype="bf16", grad_bf16=True)


def test_full_encoder_training_reduced_precision():
    # the full training workload with bf16 values, binary16 locations and
    # weights, bf16 grad_value
    w = wl.WORKLOADS["encoder_train"].scaled(value_dtype="bf16")
    core_case(w, half_locations=True, value_dtype="bf16", grad_bf16=True)


def test_f16_value_fused_front_end():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    w = wl.Workload("f16_fused", B=2, M=4, D=16, K=3, shapes=SMALL_PYRAMID[:3], ref="uniform",
                    sigma_px=2.0, Nq=33, value_dtype="f16", seed=540)
    x = wl.generate(w)
    value = torch.from_numpy(x["value_f16"]).to(dev)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("spatial_shapes", "level_start_index", "reference_points_levels",
                   "sampling_offsets", "attention_logits", "grad_output")}
    a = (value, t["spatial_shapes"], t["level_start_index"], t["reference_points_levels"],
         t["sampling_offsets"], t["attention_logits"])
    out = msda.msda_forward_fused(*a)
    gv, gr, go, gz = msda.msda_backward_fused(*a, t["grad_output"])
    torch.cuda.synchronize()
    oa = (x["value"], x["spatial_shapes"], x["level_start_index"], x["reference_points_levels"],
          x["sampling_offsets"], x["attention_logits"])
    ref, ref_abs = oracle.forward_fused(*oa, with_abs=True)
    check("output", out.cpu().numpy(), ref, ref_abs, RTOL)
    res = oracle.backward_fused(*oa, x["grad_output"], with_abs=True)
    for name, g, r, s in zip(("grad_value", "grad_ref", "grad_off", "grad_logits"),
                             (gv, gr, go, gz), res[:4], res[4:]):
        check(name, g.cpu().numpy(), r, s, RTOL)


def test_f16_input_dcn():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    w = wl.DcnWorkload("f16_dcn", B=2, H=9, W=12, G=2, D=16, sigma_px=1.5, value_dtype="f16",
                       seed=550)
    x = wl.generate_dcn(w)
    inp = torch.from_numpy(x["input_f16"]).to(dev)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("offset", "mask", "grad_output")}
    geo = dict(kernel=w.kernel, stride=w.stride, pad=w.pad, dilation=w.dilation)
    out = msda.msda_dcn_forward(inp, t["offset"], t["mask"], **geo)
    gi, go, gm = msda.msda_dcn_backward(inp, t["offset"], t["mask"], t["grad_output"], **geo)
    torch.cuda.synchronize()
    ref, ref_abs = oracle.dcn_forward(x["input"], x["offset"], x["mask"], with_abs=True, **geo)
    check("output", out.cpu().numpy(), ref, ref_abs, RTOL)
    rgi, rgo, rgm, agi, ago, agm = oracle.dcn_backward(x["input"], x["offset"], x["mask"],
                                                       x["grad_output"], with_abs=True, **geo)
    check("grad_input", gi.cpu().numpy(), rgi, agi, RTOL)
    check("grad_offset", go.cpu().numpy(), rgo, ago, RTOL)
    check("grad_mask", gm.cpu().numpy(), rgm, agm, RTOL)


def test_autograd_bf16_value_gets_bf16_gradient():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    w = wl.WORKLOADS["tiny"].scaled(value_dtype="bf16")
    x = wl.generate(w)
    v = torch.from_numpy(x["value_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    v.requires_grad_(True)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("spatial_shapes", "level_start_index", "sampling_locations",
                   "attention_weights", "grad_output")}
    out = msda.ms_deform_attn(v, t["spatial_shapes"], t["level_start_index"],
                              t["sampling_locations"], t["attention_weights"])
    (out * t["grad_output"]).sum().backward()
    assert v.grad.dtype == torch.bfloat16
    rgv, _, _, agv, _, _ = oracle.backward(x["value"], x["spatial_shapes"],
                                           x["level_start_index"], x["sampling_locations"],
                                           x["attention_weights"], x["grad_output"],
                                           with_abs=True)
    check("autograd bf16 grad_value", bf16_tensor_to_f64(v.grad), rgv, agv, RTOL_BF16_OUT)
