"""GPU parity of the fused front-end (sampling locations formed from reference
points and pixel offsets, attention weights from a softmax of logits, both
inside the kernels) against the CPU oracle's fused functions, element by
element, on the same seeded raw draws.

Tolerance as for the core (per element, r = oracle, x = GPU, S = the oracle's
sum of absolute terms): |x - r| <= rtol * |r| + 1e-5 * S with rtol 1e-5 for
fp32 values and 2e-2 for bf16 values. Both sides form the location in single
precision (the quotient offset / size rounded, then the sum rounded), so they
sample at the same point; the softmax is double in the oracle and single on
the GPU, a relative difference of a few units of 2^-24 in every weight, well
inside the S term. One more absolute term, ATOL = 1e-30, covers weights
below single precision's normal range (about 1.2e-38), which the GPU holds as
subnormals or zero while the oracle keeps them in double: such a weight's
whole contribution is below 1e-30.
"""
import numpy as np
import pytest

import oracle
from scale_deformable_attention_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 2e-2}
STOL = 1e-5
ATOL = 1e-30
SMALL_PYRAMID = ((13, 21), (7, 11), (4, 6), (2, 3))
GRADS = ("grad_value", "grad_reference_points", "grad_sampling_offsets",
         "grad_attention_logits")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scale_deformable_attention_amd as msda
    msda.library()   # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def to_gpu(x, value_dtype):
    dev = _dev()
    if value_dtype == "bf16":
        value = torch.from_numpy(x["value_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        value = torch.from_numpy(x["value"]).to(dev)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("spatial_shapes", "level_start_index", "reference_points_levels",
                   "sampling_offsets", "attention_logits", "grad_output")}
    t["value"] = value
    return t


def args(t):
    return (t["value"], t["spatial_shapes"], t["level_start_index"],
            t["reference_points_levels"], t["sampling_offsets"], t["attention_logits"])


def oracle_args(x):
    return (x["value"], x["spatial_shapes"], x["level_start_index"],
            x["reference_points_levels"], x["sampling_offsets"], x["attention_logits"])


def gpu_forward(t):
    import scale_deformable_attention_amd as msda
    out = msda.msda_forward_fused(*args(t))
    torch.cuda.synchronize()
    return out


def gpu_backward(t, needs=(True, True, True, True)):
    import scale_deformable_attention_amd as msda
    res = msda.msda_backward_fused(*args(t), t["grad_output"], needs=needs)
    torch.cuda.synchronize()
    return res


def check(name, got, ref, ref_abs, rtol):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + STOL * ref_abs + ATOL
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(
            f"{name}: {bad.sum()} of {bad.size} elements outside tolerance; first at flat "
            f"{i.tolist()}: gpu {got.reshape(-1)[i]} oracle {ref.reshape(-1)[i]} "
            f"abs-sum {ref_abs.reshape(-1)[i]}")
    # report the worst relative error where the absolute floor plays no part
    denom = np.abs(ref) + ref_abs
    big = denom > 1e-20
    rel = float(np.max(err[big] / denom[big])) if big.any() else 0.0
    print(f"  {name}: max |gpu-oracle| / (|r| + S) = {rel:.2e} "
          f"({int((~big).sum())} elements below 1e-20)", flush=True)


def parity(w, x=None, backward=True):
    print(f"[fused parity] {w.name}: B={w.B} M={w.M} D={w.D} L={w.L} K={w.K} "
          f"Nq={w.num_queries} {w.value_dtype} shapes={w.shapes}", flush=True)
    x = x if x is not None else wl.generate(w)
    t = to_gpu(x, w.value_dtype)
    rtol = RTOL[w.value_dtype]
    out = gpu_forward(t).cpu().numpy()
    ref, ref_abs = oracle.forward_fused(*oracle_args(x), with_abs=True)
    check("output", out, ref, ref_abs, rtol)
    if backward:
        got = [g.cpu().numpy() for g in gpu_backward(t)]
        res = oracle.backward_fused(*oracle_args(x), x["grad_output"], with_abs=True)
        for name, g, r, a in zip(GRADS, got, res[:4], res[4:]):
            check(name, g, r, a, rtol)
    return x, t


def test_staged_levels():
    """A plane of 2500 queries: the forward and point kernels with the coarse
    levels in LDS."""
    w = wl.Workload("fused_staged", B=1, M=2, D=32, K=4,
                    shapes=((64, 96), (32, 48), (16, 24), (8, 12)), ref="uniform",
                    sigma_px=3.0, Nq=2500, seed=192)
    parity(w, x=perturb_levels(wl.generate(w), 193))


def test_backward_in_passes():
    """A workspace holding the fixed part and the bins of 3 of the 16 (b, m)
    planes: the value gradient runs in passes; all four gradients match."""
    import bin_plan
    import scale_deformable_attention_amd as msda
    w = wl.Workload("fused_passes", B=2, M=8, D=32, K=4, shapes=SMALL_PYRAMID, ref="grid",
                    sigma_px=3.0, seed=190)
    x = perturb_levels(wl.generate(w), 191)
    t = to_gpu(x, "f32")
    full = msda.msda_backward_fused_workspace_size(t["value"], t["sampling_offsets"])
    core = bin_plan.workspace_bytes(w.B, w.M, w.num_queries, w.L, w.K, w.Nv)
    nbytes = full - core + bin_plan.workspace_bytes(w.B, w.M, w.num_queries, w.L, w.K, w.Nv,
                                                    planes=3)
    print(f"[fused parity] {w.name}: {nbytes} of {full} B of workspace", flush=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=t["value"].device)
    got = msda.msda_backward_fused(*args(t), t["grad_output"], workspace=ws)
    torch.cuda.synchronize()
    res = oracle.backward_fused(*oracle_args(x), x["grad_output"], with_abs=True)
    for name, g, r, a in zip(GRADS, [g.cpu().numpy() for g in got], res[:4], res[4:]):
        check(name, g, r, a, RTOL["f32"])


def perturb_levels(x, seed, scale=0.02):
    """Give every level its own reference point (a small shift per level)."""
    rng = np.random.default_rng(seed)
    r = x["reference_points_levels"]
    x["reference_points_levels"] = (r + rng.normal(0, scale, r.shape)).astype(np.float32)
    return x


# ---------------------------------------------------------------- small cases
def test_tiny_workload():
    parity(wl.WORKLOADS["tiny"])


@pytest.mark.parametrize("value_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_every_head_width(D, value_dtype):
    # ragged: tuple count not a multiple of any block's tuples, L*K = 9 not a
    # multiple of the lanes per tuple; per-level reference points differ
    w = wl.Workload(f"fused_D{D}_{value_dtype}", B=3, M=5, D=D, K=3, shapes=SMALL_PYRAMID[:3],
                    ref="uniform", sigma_px=2.0, Nq=37, value_dtype=value_dtype, seed=177 + D)
    parity(w, x=perturb_levels(wl.generate(w), seed=D))


def test_encoder_pyramid_small_grid():
    w = wl.Workload("fused_small_encoder", B=2, M=8, D=32, K=4, shapes=SMALL_PYRAMID,
                    ref="grid", sigma_px=3.0, seed=178)
    parity(w)


def test_single_level_single_point():
    # one weight per (query, head): the softmax is exactly 1
    w = wl.Workload("fused_single", B=2, M=1, D=16, K=1, shapes=((9, 14),), ref="uniform",
                    sigma_px=5.0, Nq=101, seed=179)
    parity(w)


def test_many_points_and_levels():
    shapes = tuple((3 + i, 2 + 2 * i) for i in range(16))
    w = wl.Workload("fused_sixteen_levels", B=1, M=2, D=8, K=5, shapes=shapes, ref="uniform",
                    sigma_px=1.5, Nq=23, seed=180)
    parity(w, x=perturb_levels(wl.generate(w), seed=5))


@pytest.mark.parametrize("i", range(6))
def test_random_configurations(i):
    # seeded draws of every size parameter, each level with its own
    # reference point
    rng = np.random.default_rng(8000 + i)
    L = int(rng.integers(1, 6))
    shapes = tuple((int(rng.integers(1, 41)), int(rng.integers(1, 71))) for _ in range(L))
    w = wl.Workload(f"fused_random_{i}", B=int(rng.integers(1, 3)), M=int(rng.integers(1, 5)),
                    D=int(rng.choice([8, 16, 32, 64])), K=int(rng.integers(1, 6)), shapes=shapes,
                    ref="uniform", sigma_px=float(rng.uniform(0.5, 12.0)),
                    Nq=int(rng.integers(1, 400)), seed=8100 + i)
    parity(w, x=perturb_levels(wl.generate(w), seed=8200 + i))


def test_extreme_logits_and_far_offsets():
    w = wl.Workload("fused_extreme", B=2, M=4, D=32, K=4, shapes=SMALL_PYRAMID, ref="uniform",
                    sigma_px=30.0, Nq=50, seed=181)
    x = wl.generate(w)
    z = x["attention_logits"]
    z[0, :, :, :] *= 40.0           # spreads of hundreds: max-shift needed, many weights 0
    z[1, ::3, :, :] = 7.5           # all equal: uniform weights
    z[1, 1::3, :, 0] = 88.0         # one dominant logit near the single-precision exp limit
    parity(w, x=x)


def test_empty_work():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    shapes = torch.tensor([[4, 4]], dtype=torch.int64, device=dev)
    lsi = torch.tensor([0], dtype=torch.int64, device=dev)
    value = torch.randn(2, 16, 2, 8, device=dev)
    # K = 0: output zeros, every gradient zero or empty
    ref = torch.rand(2, 5, 1, 2, device=dev)
    off = torch.rand(2, 5, 2, 1, 0, 2, device=dev)
    z = torch.rand(2, 5, 2, 0, device=dev)
    out = msda.msda_forward_fused(value, shapes, lsi, ref, off, z)
    gv, gr, go, gz = msda.msda_backward_fused(value, shapes, lsi, ref, off, z,
                                              torch.randn(2, 5, 16, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (2, 5, 16) and torch.all(out == 0)
    assert torch.all(gv == 0) and torch.all(gr == 0) and go.numel() == 0 and gz.numel() == 0
    # B = 0
    value0 = torch.randn(0, 16, 2, 8, device=dev)
    ref0 = torch.rand(0, 5, 1, 2, device=dev)
    off0 = torch.rand(0, 5, 2, 1, 3, 2, device=dev)
    z0 = torch.rand(0, 5, 2, 3, device=dev)
    out0 = msda.msda_forward_fused(value0, shapes, lsi, ref0, off0, z0)
    g0 = msda.msda_backward_fused(value0, shapes, lsi, ref0, off0, z0,
                                  torch.zeros(0, 5, 16, device=dev))
    torch.cuda.synchronize()
    assert out0.numel() == 0 and all(g.numel() == 0 for g in g0)
    # Nq = 0: grad_value still zeroed
    refq = torch.rand(2, 0, 1, 2, device=dev)
    offq = torch.rand(2, 0, 2, 1, 3, 2, device=dev)
    zq = torch.rand(2, 0, 2, 3, device=dev)
    out = msda.msda_forward_fused(value, shapes, lsi, refq, offq, zq)
    gv, gr, go, gz = msda.msda_backward_fused(value, shapes, lsi, refq, offq, zq,
                                              torch.zeros(2, 0, 16, device=dev))
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.all(gv == 0) and gr.numel() == 0


def test_skipped_gradients_match_full_call():
    w = wl.Workload("fused_skip", B=2, M=4, D=16, K=3, shapes=SMALL_PYRAMID[:3],
                    ref="uniform", sigma_px=2.0, Nq=29, seed=182)
    x = perturb_levels(wl.generate(w), seed=9)
    t = to_gpu(x, "f32")
    full = gpu_backward(t)
    for i in range(4):
        needs = tuple(j == i for j in range(4))
        got = gpu_backward(t, needs=needs)
        for j, (g, r) in enumerate(zip(got, full)):
            if j == i:
                # the reference-point gradient alone runs through a workspace
                # copy of the offset gradient: same numbers
                assert torch.allclose(g, r, rtol=1e-6, atol=1e-6), GRADS[i]
            else:
                assert g is None
    got = gpu_backward(t, needs=(False, True, False, True))
    assert torch.allclose(got[1], full[1], rtol=1e-6, atol=1e-6)
    assert torch.allclose(got[3], full[3], rtol=1e-6, atol=1e-6)


def test_fused_matches_core_on_the_same_locations():
    # the fused forward equals the core forward fed the locations and weights
    # formed on the host in the same precision (single: quotient, then sum;
    # weights from the oracle's double softmax rounded): both GPU paths agree
    w = wl.Workload("fused_vs_core", B=2, M=8, D=32, K=4, shapes=SMALL_PYRAMID, ref="uniform",
                    sigma_px=2.5, Nq=64, seed=183)
    x = wl.generate(w)
    t = to_gpu(x, "f32")
    import scale_deformable_attention_amd as msda
    fused = gpu_forward(t)
    shapes = x["spatial_shapes"]
    wh = np.stack([shapes[:, 1], shapes[:, 0]], -1).astype(np.float32)         # (W, H)
    q = (x["sampling_offsets"] / wh[None, None, None, :, None, :]).astype(np.float32)
    loc = (x["reference_points_levels"][:, :, None, :, None, :] + q).astype(np.float32)
    z = x["attention_logits"].astype(np.float64)
    e = np.exp(z - z.max(-1, keepdims=True))
    attn = (e / e.sum(-1, keepdims=True)).astype(np.float32).reshape(loc.shape[:-1])
    dev = t["value"].device
    core = msda.msda_forward(t["value"], t["spatial_shapes"], t["level_start_index"],
                             torch.from_numpy(loc).to(dev), torch.from_numpy(attn).to(dev))
    torch.cuda.synchronize()
    np.testing.assert_allclose(fused.cpu().numpy(), core.cpu().numpy(), rtol=1e-5, atol=2e-6)


def test_outputs_are_overwritten_and_deterministic():
    w = wl.WORKLOADS["tiny"]
    x = wl.generate(w)
    t = to_gpu(x, "f32")
    a = gpu_forward(t)
    b = gpu_forward(t)
    assert torch.equal(a, b)
    g1 = gpu_backward(t)
    import scale_deformable_attention_amd as msda
    g2 = [torch.full_like(g, 77.0) for g in g1]
    msda.msda_backward_fused(*args(t), t["grad_output"], grad_value=g2[0],
                             grad_reference_points=g2[1], grad_sampling_offsets=g2[2],
                             grad_attention_logits=g2[3])
    torch.cuda.synchronize()
    # the point gradients are formed per point: bitwise repeatable; grad_value
    # sums a pixel's entries in the order the binning placed them
    assert torch.allclose(g1[0], g2[0], rtol=1e-6, atol=1e-6)
    for u, v in zip(g1[1:], g2[1:]):
        assert torch.equal(u, v)


def test_autograd_function_matches_oracle():
    import scale_deformable_attention_amd as msda
    w = wl.WORKLOADS["tiny"]
    x = perturb_levels(wl.generate(w), seed=11)
    t = to_gpu(x, "f32")
    v = t["value"].clone().requires_grad_(True)
    r = t["reference_points_levels"].clone().requires_grad_(True)
    o = t["sampling_offsets"].clone().requires_grad_(True)
    z = t["attention_logits"].clone().requires_grad_(True)
    out = msda.ms_deform_attn_fused(v, t["spatial_shapes"], t["level_start_index"], r, o, z)
    (out * t["grad_output"]).sum().backward()
    res = oracle.backward_fused(*oracle_args(x), x["grad_output"], with_abs=True)
    for name, g, ref, a in zip(GRADS, (v.grad, r.grad, o.grad, z.grad), res[:4], res[4:]):
        check("autograd " + name, g.cpu().numpy(), ref, a, 1e-5)


# ---------------------------------------------------------------- full size
def test_full_encoder_training_step_fused():
    parity(wl.WORKLOADS["encoder_train"])


def test_full_decoder_fused():
    parity(wl.WORKLOADS["decoder"])
