"""The allocation-free backward (msda_backward_noalloc, through the C ABI)
against msda_backward with a workspace, on two calls in a row, the second with
a smaller input than the first (the static scratch then holds the first call's
contents). The location and weight gradients sum in a fixed order and must be
bitwise equal; grad_value (whose summation order follows LDS atomics) must
agree within the parity tolerance, |x - y| <= 1e-5 (|r| + S) with r and S from
the oracle, and both must match the oracle."""
import numpy as np
import pytest

import oracle
from scale_deformable_attention_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scale_deformable_attention_amd as msda
    msda.library()
    return torch.device("cuda:0")


def _inputs(w, dev):
    x = wl.generate(w)
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
         for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                   "attention_weights", "grad_output")}
    return x, t


def _args(t):
    return (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
            t["attention_weights"], t["grad_output"])


def _compare(w, x, got, ref_ws):
    rgv, rgl, rga, agv, agl, aga = oracle.backward(
        x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
        x["attention_weights"], x["grad_output"], with_abs=True)
    gv, gl, ga = [g.cpu().numpy().astype(np.float64) for g in got]
    wv, wl_, wa = [g.cpu().numpy().astype(np.float64) for g in ref_ws]
    assert np.array_equal(gl, wl_), f"{w.name}: location gradients differ between entry points"
    assert np.array_equal(ga, wa), f"{w.name}: weight gradients differ between entry points"
    gv, wv = gv.reshape(rgv.shape), wv.reshape(rgv.shape)
    bound = TOL * (np.abs(rgv) + agv)
    assert np.all(np.abs(gv - wv) <= bound), f"{w.name}: grad_value differs between entry points"
    for name, g, r, s in (("grad_value", gv, rgv, agv), ("grad_loc", gl.reshape(rgl.shape), rgl, agl),
                          ("grad_attn", ga.reshape(rga.shape), rga, aga)):
        assert np.all(np.abs(g - r) <= TOL * (np.abs(r) + s)), f"{w.name}: {name} vs oracle"
    print(f"[noalloc] {w.name}: matches msda_backward and the oracle", flush=True)


def test_noalloc_matches_backward_on_two_calls():
    import scale_deformable_attention_amd as msda
    dev = _dev()
    big = wl.Workload("noalloc_big", B=2, M=8, D=32, K=4,
                      shapes=((13, 21), (7, 11), (4, 6), (2, 3)), ref="grid", sigma_px=3.0,
                      seed=950)
    small = wl.WORKLOADS["tiny"]
    xb, tb = _inputs(big, dev)
    xs, ts = _inputs(small, dev)
    assert msda.msda_backward_workspace_size(tb["value"], tb["sampling_locations"]) > \
        msda.msda_backward_workspace_size(ts["value"], ts["sampling_locations"])
    print(f"[noalloc] {big.name} then {small.name}", flush=True)
    got_b = msda.msda_backward_noalloc(*_args(tb))
    got_s = msda.msda_backward_noalloc(*_args(ts))      # second call, smaller input
    torch.cuda.synchronize()
    ref_b = msda.msda_backward(*_args(tb))
    ref_s = msda.msda_backward(*_args(ts))
    torch.cuda.synchronize()
    _compare(big, xb, got_b, ref_b)
    _compare(small, xs, got_s, ref_s)


def test_noalloc_runs_a_large_problem_in_passes():
    """A problem whose bins exceed the static scratch but whose single (b, m)
    planes fit runs in several passes over the planes."""
    import bin_plan
    import scale_deformable_attention_amd as msda
    dev = _dev()
    w = wl.Workload("noalloc_passes", B=2, M=8, D=32, K=4,
                    shapes=((50, 84), (25, 42), (13, 21), (7, 11)), ref="uniform",
                    sigma_px=3.0, Nq=5000, seed=951)
    full = bin_plan.workspace_bytes(w.B, w.M, w.num_queries, w.L, w.K, w.Nv)
    assert full > msda._binding.NOALLOC_SCRATCH_BYTES
    assert bin_plan.workspace_bytes(w.B, w.M, w.num_queries, w.L, w.K, w.Nv, planes=1) < \
        msda._binding.NOALLOC_SCRATCH_BYTES
    x, t = _inputs(w, dev)
    print(f"[noalloc] {w.name}: {full / 2**20:.0f} MiB of bins in passes", flush=True)
    got = msda.msda_backward_noalloc(*_args(t))
    torch.cuda.synchronize()
    ref = msda.msda_backward(*_args(t))
    torch.cuda.synchronize()
    _compare(w, x, got, ref)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """One (b, m) plane's bins larger than the scratch: refused, nothing written."""
    import bin_plan
    import scale_deformable_attention_amd as msda
    dev = _dev()
    B, Nv, M, D, L, K, Nq = 1, 22223, 1, 32, 4, 4, 100000
    assert bin_plan.workspace_bytes(B, M, Nq, L, K, Nv, planes=1) > \
        msda._binding.NOALLOC_SCRATCH_BYTES
    value = torch.zeros(B, Nv, M, D, device=dev)
    shapes = torch.tensor([[100, 167], [50, 84], [25, 42], [13, 21]], dtype=torch.int64,
                          device=dev)
    lsi = torch.tensor([0, 16700, 20900, 21950], dtype=torch.int64, device=dev)
    loc = torch.full((B, Nq, M, L, K, 2), 0.5, device=dev)
    attn = torch.full((B, Nq, M, L, K), 0.25, device=dev)
    g = torch.ones(B, Nq, M * D, device=dev)
    gv = torch.full((B, Nv, M, D), 7.0, device=dev)
    with pytest.raises(msda.MsdaError) as e:
        msda.msda_backward_noalloc(value, shapes, lsi, loc, attn, g, grad_value=gv)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((gv == 7.0).all()), "a refused call wrote grad_value"
    # without grad_value no scratch is needed: the call goes through
    _, gl, ga = msda.msda_backward_noalloc(value, shapes, lsi, loc, attn, g,
                                           needs=(False, True, True))
    torch.cuda.synchronize()
    assert gl is not None and ga is not None
