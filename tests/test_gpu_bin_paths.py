"""GPU parity of the value gradient through the plain (not register-cached) bin
kernel, on every front-end that bins normalized locations, with 4-row and
8-row tiles.

The backward picks the register-cached bin kernel whenever every bin block can
keep its points in registers without more than tripling the block count; with
many points per query (L*K = 128) and few blocks per (b, m) it cannot, and the
plain kernel loads each point once per pass instead. Each case asserts (with the
plan restated in tests/bin_plan.py, itself checked against the library's
workspace size) that it takes that kernel, then compares every gradient with the
oracle at the same tolerances as the other parity tests.
"""
import numpy as np
import pytest

import bin_plan
import test_gpu_fused as fused
import test_gpu_parity as core
import test_gpu_precision as precision
from scale_deformable_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

SMALL = ((10, 12), (5, 6), (3, 3), (2, 2))          # Nv = 163: points outnumber pixels
LARGE = ((128, 128), (64, 64), (32, 32), (16, 16))  # Nv = 21760: pixels outnumber points


def _plain_kernel(w, tall):
    nW, Qc, cached, is_tall = bin_plan.plan(w.B, w.M, w.num_queries, w.L, w.K, w.Nv)
    assert not cached, f"{w.name} would take the register-cached bin kernel"
    assert is_tall == tall, f"{w.name}: tall tiles {is_tall}"
    print(f"[bin plan] {w.name}: {nW} plain bin blocks per (b, m) of {Qc} queries, "
          f"{'8' if tall else '4'}-row tiles", flush=True)


@pytest.mark.parametrize("D", [8, 16, 32, 64])
def test_core_plain_bin_kernel(D):
    w = wl.Workload(f"plain_bin_D{D}", B=1, M=2, D=D, K=32, shapes=SMALL, ref="uniform",
                    sigma_px=1.5, Nq=256, seed=900 + D)
    _plain_kernel(w, tall=False)
    core.parity(w)


@pytest.mark.parametrize("D", [16, 32])
def test_core_plain_bin_kernel_tall_tiles(D):
    w = wl.Workload(f"plain_bin_tall_D{D}", B=1, M=2, D=D, K=32, shapes=LARGE, ref="uniform",
                    sigma_px=2.0, Nq=100, seed=910 + D)
    _plain_kernel(w, tall=True)
    core.parity(w)


def test_core_plain_bin_kernel_bf16_value():
    w = wl.Workload("plain_bin_bf16", B=1, M=2, D=32, K=32, shapes=SMALL, ref="uniform",
                    sigma_px=1.5, Nq=256, value_dtype="bf16", seed=920)
    _plain_kernel(w, tall=False)
    core.parity(w)


def test_fused_plain_bin_kernel():
    w = wl.Workload("plain_bin_fused", B=1, M=2, D=32, K=32, shapes=SMALL, ref="uniform",
                    sigma_px=1.5, Nq=256, seed=930)
    _plain_kernel(w, tall=False)
    fused.parity(w, x=fused.perturb_levels(wl.generate(w), 931))


def test_fused_plain_bin_kernel_tall_tiles():
    w = wl.Workload("plain_bin_fused_tall", B=1, M=2, D=16, K=32, shapes=LARGE, ref="uniform",
                    sigma_px=2.0, Nq=100, seed=932)
    _plain_kernel(w, tall=True)
    fused.parity(w)


def test_half_locations_plain_bin_kernel():
    w = wl.Workload("plain_bin_hloc", B=1, M=2, D=32, K=32, shapes=SMALL, ref="uniform",
                    sigma_px=1.5, Nq=256, seed=940)
    _plain_kernel(w, tall=False)
    precision.core_case(w, half_locations=True, value_dtype="f32", grad_bf16=False)


def test_half_locations_plain_bin_kernel_tall_tiles():
    w = wl.Workload("plain_bin_hloc_tall", B=1, M=2, D=16, K=32, shapes=LARGE, ref="uniform",
                    sigma_px=2.0, Nq=100, seed=942)
    _plain_kernel(w, tall=True)
    precision.core_case(w, half_locations=True, value_dtype="f32", grad_bf16=False)
