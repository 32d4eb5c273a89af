"""GPU parity of the grouped single-level deformable aggregation (DCNv3)
against the CPU oracle (oracle.dcn_forward / dcn_backward), element by
element, through the C ABI.

Tolerance as for the core: |x - r| <= rtol * |r| + 1e-5 * S, rtol 1e-5 for
fp32 inputs and 2e-2 for bf16 inputs (the oracle is fed the same bf16
values), S = the oracle's sum of the absolute values of the element's terms.
Both sides form the sampling point in single precision (grid coordinate plus
offset, one rounding), so they sample at the same point.
"""
import numpy as np
import pytest

import oracle
from scale_deformable_attention_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 2e-2}
STOL = 1e-5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scale_deformable_attention_amd as msda
    msda.library()   # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def check(name, got, ref, ref_abs, rtol):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= rtol * np.abs(ref) + STOL * ref_abs)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(
            f"{name}: {bad.sum()} of {bad.size} elements outside tolerance; first at flat "
            f"{i.tolist()}: gpu {got.reshape(-1)[i]} oracle {ref.reshape(-1)[i]} "
            f"abs-sum {ref_abs.reshape(-1)[i]}")
    denom = np.abs(ref) + ref_abs
    big = denom > 0
    rel = float(np.max(err[big] / denom[big])) if big.any() else 0.0
    print(f"  {name}: max |gpu-oracle| / (|r| + S) = {rel:.2e}", flush=True)


def to_gpu(x, w):
    dev = _dev()
    if w.value_dtype == "bf16":
        inp = torch.from_numpy(x["input_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        inp = torch.from_numpy(x["input"]).to(dev)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("offset", "mask", "grad_output")}
    t["input"] = inp
    return t


def geometry(w):
    return dict(kernel=w.kernel, stride=w.stride, pad=w.pad, dilation=w.dilation)


def parity(w, x=None, backward=True):
    import scale_deformable_attention_amd as msda
    print(f"[dcn parity] {w.name}: B={w.B} H={w.H} W={w.W} G={w.G} D={w.D} kernel={w.kernel} "
          f"stride={w.stride} pad={w.pad} dilation={w.dilation} out={w.out_size} "
          f"{w.value_dtype}", flush=True)
    x = x if x is not None else wl.generate_dcn(w)
    t = to_gpu(x, w)
    geo = geometry(w)
    rtol = RTOL[w.value_dtype]
    out = msda.msda_dcn_forward(t["input"], t["offset"], t["mask"], **geo)
    torch.cuda.synchronize()
    ref, ref_abs = oracle.dcn_forward(x["input"], x["offset"], x["mask"], with_abs=True, **geo)
    check("output", out.cpu().numpy(), ref, ref_abs, rtol)
    if backward:
        gi, go, gm = msda.msda_dcn_backward(t["input"], t["offset"], t["mask"], t["grad_output"],
                                            **geo)
        torch.cuda.synchronize()
        rgi, rgo, rgm, agi, ago, agm = oracle.dcn_backward(
            x["input"], x["offset"], x["mask"], x["grad_output"], with_abs=True, **geo)
        check("grad_input", gi.cpu().numpy(), rgi, agi, rtol)
        check("grad_offset", go.cpu().numpy(), rgo, ago, rtol)
        check("grad_mask", gm.cpu().numpy(), rgm, agm, rtol)
    return x, t


def test_backward_in_passes():
    """A workspace holding one (b, group) plane's bins: the input gradient runs
    in passes over the planes and matches the oracle."""
    import bin_plan
    import scale_deformable_attention_amd as msda
    w = wl.DcnWorkload("dcn_passes", B=2, H=12, W=14, G=4, D=16, sigma_px=1.5, seed=450)
    x = wl.generate_dcn(w)
    t = to_gpu(x, w)
    geo = geometry(w)
    Ho, Wo = w.out_size
    K = w.kernel[0] * w.kernel[1]
    nbytes = bin_plan.workspace_bytes(w.B, w.G, Ho * Wo, 1, K, w.H * w.W, planes=1)
    print(f"[dcn parity] {w.name}: {nbytes} B of workspace, one plane per pass", flush=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=t["input"].device)
    gi, go, gm = msda.msda_dcn_backward(t["input"], t["offset"], t["mask"], t["grad_output"],
                                        workspace=ws, **geo)
    torch.cuda.synchronize()
    rgi, rgo, rgm, agi, ago, agm = oracle.dcn_backward(
        x["input"], x["offset"], x["mask"], x["grad_output"], with_abs=True, **geo)
    check("grad_input", gi.cpu().numpy(), rgi, agi, RTOL["f32"])
    check("grad_offset", go.cpu().numpy(), rgo, ago, RTOL["f32"])
    check("grad_mask", gm.cpu().numpy(), rgm, agm, RTOL["f32"])


def test_tiny():
    parity(wl.DCN_WORKLOADS["dcn_tiny"])


@pytest.mark.parametrize("value_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_every_group_width(D, value_dtype):
    w = wl.DcnWorkload(f"dcn_D{D}_{value_dtype}", B=2, H=9, W=11, G=3, D=D, sigma_px=1.5,
                       value_dtype=value_dtype, seed=400 + D)
    parity(w)


@pytest.mark.parametrize("kernel,stride,pad,dilation", [
    ((3, 3), (2, 2), (1, 1), (1, 1)), ((5, 3), (1, 2), (4, 1), (2, 1)),
    ((3, 2), (2, 1), (2, 3), (1, 3)), ((1, 1), (1, 1), (0, 0), (1, 1)),
    ((7, 7), (1, 1), (3, 3), (1, 1)),
    # fewer points than input pixels: the 8-row grad_value tiles
    ((1, 1), (2, 2), (0, 0), (1, 1))])
def test_grid_geometries(kernel, stride, pad, dilation):
    w = wl.DcnWorkload(f"dcn_{kernel}_{stride}_{pad}_{dilation}", B=2, H=13, W=10, G=2, D=16,
                       kernel=kernel, stride=stride, pad=pad, dilation=dilation, sigma_px=1.0,
                       seed=410 + kernel[0] * 7 + stride[1])
    parity(w)


def random_dcn(i):
    rng = np.random.default_rng(9000 + i)
    while True:
        k = (int(rng.integers(1, 6)), int(rng.integers(1, 6)))
        w = wl.DcnWorkload(f"dcn_random_{i}", B=int(rng.integers(1, 3)),
                           H=int(rng.integers(1, 30)), W=int(rng.integers(1, 40)),
                           G=int(rng.integers(1, 5)), D=int(rng.choice([8, 16, 32, 64])),
                           kernel=k, stride=(int(rng.integers(1, 4)), int(rng.integers(1, 4))),
                           pad=(int(rng.integers(0, 4)), int(rng.integers(0, 4))),
                           dilation=(int(rng.integers(1, 4)), int(rng.integers(1, 4))),
                           sigma_px=float(rng.uniform(0.3, 4.0)), seed=9100 + i)
        if min(w.out_size) >= 1:
            return w


@pytest.mark.parametrize("i", range(6))
def test_random_configurations(i):
    # seeded draws of the sizes and of the grid geometry
    parity(random_dcn(i))


def test_far_and_non_finite_offsets():
    w = wl.DcnWorkload("dcn_far", B=1, H=12, W=15, G=4, D=16, sigma_px=25.0, seed=420)
    x = wl.generate_dcn(w)
    flat = x["offset"].reshape(-1, 2)
    flat[0::7, 0] = np.nan
    flat[3::11, 1] = np.inf
    flat[5::13, 0] = -np.inf
    flat[6::17] = 1e30
    parity(w, x=x)


def test_empty_work():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    # no output pixels (a 3x3 grid does not fit a 2-row unpadded input)
    inp = torch.randn(1, 2, 5, 2, 8, device=dev)
    off = torch.zeros(1, 0, 3, 2, 9, 2, device=dev)
    mask = torch.zeros(1, 0, 3, 2, 9, device=dev)
    out = msda.msda_dcn_forward(inp, off, mask, (3, 3))
    gi = torch.full_like(inp, 5.0)
    msda.msda_dcn_backward(inp, off, mask, torch.zeros(1, 0, 3, 16, device=dev), (3, 3),
                           grad_input=gi)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.all(gi == 0)
    # B = 0
    inp0 = torch.randn(0, 4, 4, 2, 8, device=dev)
    off0 = torch.zeros(0, 4, 4, 2, 9, 2, device=dev)
    m0 = torch.zeros(0, 4, 4, 2, 9, device=dev)
    out0 = msda.msda_dcn_forward(inp0, off0, m0, (3, 3), pad=(1, 1))
    g0 = msda.msda_dcn_backward(inp0, off0, m0, torch.zeros(0, 4, 4, 16, device=dev), (3, 3),
                                pad=(1, 1))
    torch.cuda.synchronize()
    assert out0.numel() == 0 and all(g.numel() == 0 for g in g0)


def test_skipped_gradients_and_overwrite():
    import scale_deformable_attention_amd as msda
    w = wl.DCN_WORKLOADS["dcn_tiny"]
    x = wl.generate_dcn(w)
    t = to_gpu(x, w)
    geo = geometry(w)
    full = msda.msda_dcn_backward(t["input"], t["offset"], t["mask"], t["grad_output"], **geo)
    for i in range(3):
        needs = tuple(j == i for j in range(3))
        got = msda.msda_dcn_backward(t["input"], t["offset"], t["mask"], t["grad_output"],
                                     needs=needs, **geo)
        for j, (g, r) in enumerate(zip(got, full)):
            if j == i:
                assert torch.allclose(g, r, rtol=1e-6, atol=1e-6)
            else:
                assert g is None
    gi = torch.full_like(full[0], 3.0)
    go = torch.full_like(full[1], -1.0)
    gm = torch.full_like(full[2], 8.0)
    msda.msda_dcn_backward(t["input"], t["offset"], t["mask"], t["grad_output"], grad_input=gi,
                           grad_offset=go, grad_mask=gm, **geo)
    torch.cuda.synchronize()
    assert torch.allclose(gi, full[0], rtol=1e-6, atol=1e-6)
    assert torch.equal(go, full[1]) and torch.equal(gm, full[2])


def test_full_stage2():
    parity(wl.DCN_WORKLOADS["dcnv3_stage2"])


def test_full_stage1():
    parity(wl.DCN_WORKLOADS["dcnv3_stage1"])
