"""GPU parity of the linear layers (matrix-core GEMMs) and of the whole
MSDeformAttn layer against the CPU oracle (oracle/layer.py), element by
element, through the C ABI.

Tolerance: |x - r| <= 1e-5 * |r| + 1e-5 * S + 1e-30, S = the oracle's sum of
the absolute values of the terms of the element, propagated through the
layer's steps. A linear layer's output is an fp32 sum of `in_features`
products (its weight gradient: of `rows` products, split over blocks and the
splits summed in order), whose rounding error is a small multiple of
2^-24 * sqrt(n) * S for these sizes.

The layer tests draw every activation and weight on a dyadic grid
(workloads.generate_layer): the offset, logit, value and upstream-gradient
projections are then exact in single precision, so the GPU and the oracle
sample at bitwise the same locations and the comparison is not exposed to a
location landing on the other side of a pixel boundary (where the location
gradient is discontinuous). One small test uses plain normal draws as well.
"""
import numpy as np
import pytest

from oracle import layer as olayer
from scale_deformable_attention_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL, STOL, ATOL = 1e-5, 1e-5, 1e-30
NAMES = {"value_weight": "w_value", "value_bias": "b_value", "offset_weight": "w_offset",
         "offset_bias": "b_offset", "attn_weight": "w_attn", "attn_bias": "b_attn",
         "output_weight": "w_out", "output_bias": "b_out"}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scale_deformable_attention_amd as msda
    msda.library()
    return torch.device("cuda:0")


def check(name, got, ref, s):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= RTOL * np.abs(ref) + STOL * s + ATOL)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{i.tolist()}: gpu {got.reshape(-1)[i]} oracle {ref.reshape(-1)[i]} "
                             f"S {s.reshape(-1)[i]}")
    denom = np.abs(ref) + s
    big = denom > 1e-20
    rel = float(np.max(err[big] / denom[big])) if big.any() else 0.0
    print(f"  {name}: max |gpu-oracle| / (|r| + S) = {rel:.2e}", flush=True)


# ---------------------------------------------------------------- linear layers
@pytest.mark.parametrize("rows,fin,fout", [(1000, 256, 256), (333, 256, 384), (130, 256, 128),
                                           (77, 13, 9), (5, 24, 40), (0, 16, 8),
                                           (2049, 64, 130)])
def test_linear_parity(rows, fin, fout):
    dev = _dev()
    import scale_deformable_attention_amd as msda
    print(f"[linear] rows={rows} in={fin} out={fout}", flush=True)
    rng = np.random.default_rng(rows * 7 + fin + fout)
    x = rng.standard_normal((rows, fin)).astype(np.float32)
    w = (rng.standard_normal((fout, fin)) / np.sqrt(fin)).astype(np.float32)
    b = rng.standard_normal(fout).astype(np.float32)
    gy = rng.standard_normal((rows, fout)).astype(np.float32)
    X, Wt, Bt, G = (torch.from_numpy(a).to(dev) for a in (x, w, b, gy))
    y = msda.msda_linear_forward(X, Wt, Bt)
    gx, gw, gb = msda.msda_linear_backward(X, Wt, G)
    torch.cuda.synchronize()
    ry, sy = olayer.linear_forward(x, w, b, with_abs=True)
    check("y", y.cpu().numpy(), ry, sy)
    rgx, rgw, rgb, sgx, sgw, sgb = olayer.linear_backward(x, w, gy, with_abs=True)
    check("grad_x", gx.cpu().numpy(), rgx, sgx)
    check("grad_weight", gw.cpu().numpy(), rgw, sgw)
    check("grad_bias", gb.cpu().numpy(), rgb, sgb)


def test_linear_without_bias_and_repeatable():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((3000, 256)).astype(np.float32)).to(dev)
    w = torch.from_numpy(rng.standard_normal((256, 256)).astype(np.float32) / 16).to(dev)
    g = torch.from_numpy(rng.standard_normal((3000, 256)).astype(np.float32)).to(dev)
    y = msda.msda_linear_forward(x, w, None)
    a = msda.msda_linear_backward(x, w, g)
    b = msda.msda_linear_backward(x, w, g)
    torch.cuda.synchronize()
    ry = olayer.linear_forward(x.cpu().numpy(), w.cpu().numpy())
    np.testing.assert_allclose(y.cpu().numpy(), ry, rtol=1e-5, atol=1e-4)
    for u, v in zip(a, b):
        assert torch.equal(u, v)   # fixed summation order


# ---------------------------------------------------------------- the layer
def _layer_inputs(x, dev):
    t = {k: torch.from_numpy(np.array(v, copy=True)).to(dev) for k, v in x.items()}
    params = {k: t[k] for k in NAMES}
    return t, params


def layer_parity(w, x=None, backward=True, skip=()):
    dev = _dev()
    import scale_deformable_attention_amd as msda
    print(f"[layer parity] {w.name}: B={w.B} M={w.M} D={w.D} L={w.L} K={w.K} "
          f"Nq={w.num_queries} Nv={w.Nv}", flush=True)
    x = x if x is not None else wl.generate_layer(w)
    t, params = _layer_inputs(x, dev)
    args = (t["query"], t["input_flatten"], t["reference_points"], t["spatial_shapes"],
            t["level_start_index"], params, w.M, w.K)
    out, saved = msda.msda_layer_forward(*args)
    g = msda.msda_layer_backward(*args, saved, t["grad_output"]) if backward else None
    torch.cuda.synchronize()
    p = {NAMES[k]: x[k] for k in NAMES}
    oargs = (p, x["query"], x["input_flatten"], x["reference_points"], x["spatial_shapes"],
             x["level_start_index"], w.M, w.L, w.K)
    ref, s = olayer.layer_forward(*oargs, with_abs=True)
    check("output", out.cpu().numpy(), ref, s)
    if backward:
        rg, sg = olayer.layer_backward(*oargs, x["grad_output"], with_abs=True)
        for k in ("query", "input_flatten", "reference_points"):
            if k not in skip:
                check("grad_" + k, g[k].cpu().numpy(), rg[k], sg[k])
        for k, ok in NAMES.items():
            if k not in skip:
                check("grad_" + k, g[k].cpu().numpy(), rg[ok], sg[ok])
    return x, t


def test_layer_tiny():
    layer_parity(wl.WORKLOADS["tiny"])


SMALL_PYRAMID = ((13, 21), (7, 11), (4, 6), (2, 3))


@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_layer_head_widths(D):
    w = wl.Workload(f"layer_D{D}", B=2, M=4, D=D, K=3, shapes=SMALL_PYRAMID[:3], ref="uniform",
                    sigma_px=2.0, Nq=45, seed=300 + D)
    layer_parity(w)


def test_layer_odd_head_sizes():
    # M*L*K = 3: the offset (6) and logit (3) features are not multiples of 4
    # (scalar operand loads) and the query gradient's two heads run as two
    # products (offset features not a multiple of 16)
    w = wl.Workload("layer_odd", B=2, M=1, D=16, K=3, shapes=((7, 9),), ref="uniform",
                    sigma_px=2.0, Nq=21, seed=320)
    layer_parity(w)


@pytest.mark.parametrize("i", range(3))
def test_layer_random_configurations(i):
    # seeded draws of heads, head width, levels and their shapes, points,
    # batch and queries (dyadic activations and weights)
    rng = np.random.default_rng(9500 + i)
    L = int(rng.integers(1, 5))
    shapes = tuple((int(rng.integers(1, 25)), int(rng.integers(1, 40))) for _ in range(L))
    w = wl.Workload(f"layer_random_{i}", B=int(rng.integers(1, 3)), M=int(rng.integers(1, 5)),
                    D=int(rng.choice([8, 16, 32])), K=int(rng.integers(1, 5)), shapes=shapes,
                    ref="uniform", sigma_px=float(rng.uniform(0.5, 6.0)),
                    Nq=int(rng.integers(1, 200)), seed=9600 + i)
    layer_parity(w)


def test_layer_small_encoder_grid():
    w = wl.Workload("layer_small_encoder", B=2, M=8, D=32, K=4, shapes=SMALL_PYRAMID, ref="grid",
                    sigma_px=3.0, seed=310)
    layer_parity(w)


def test_layer_normal_draws():
    # Plain (non-dyadic) draws at a small size. The offset projection is then
    # rounded differently on the two sides (single-precision sums in another
    # order), so the sampling locations differ by an ulp or two: a bilinear
    # weight moves by ~1e-7 absolute. The output and the gradients that sum
    # the weights of a sample's four corners do not notice; a value-gradient
    # pixel reached only through small corner weights sees it as a relative
    # change above 1e-5 of its own terms. That gradient (and the input
    # gradient built from it) is compared on the dyadic cases above, where the
    # locations are bitwise equal; here the rest is.
    w = wl.Workload("layer_normal", B=1, M=2, D=8, K=2, shapes=((6, 9), (3, 5)), ref="uniform",
                    sigma_px=2.0, Nq=20, seed=311)
    x = wl.generate_layer(w)
    rng = np.random.default_rng(312)
    for k, v in list(x.items()):
        if v.dtype == np.float32 and k != "reference_points":
            x[k] = (v + rng.standard_normal(v.shape).astype(np.float32) * 1e-3 *
                    (np.abs(v).max() + 1e-3)).astype(np.float32)
    layer_parity(w, x=x, skip=("input_flatten", "value_weight", "value_bias"))


def test_layer_only_some_gradients():
    dev = _dev()
    import scale_deformable_attention_amd as msda
    w = wl.WORKLOADS["tiny"]
    x = wl.generate_layer(w)
    t, params = _layer_inputs(x, dev)
    args = (t["query"], t["input_flatten"], t["reference_points"], t["spatial_shapes"],
            t["level_start_index"], params, w.M, w.K)
    out, saved = msda.msda_layer_forward(*args)
    full = msda.msda_layer_backward(*args, saved, t["grad_output"])
    part = msda.msda_layer_backward(*args, saved, t["grad_output"],
                                    needs_inputs=(True, False, False), needs_params=False)
    torch.cuda.synchronize()
    assert set(part) == {"query"}
    assert torch.equal(part["query"], full["query"])


def test_full_encoder_training_layer():
    layer_parity(wl.WORKLOADS["encoder_train"])
