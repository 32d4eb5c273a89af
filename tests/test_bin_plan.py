"""The test-side restatement of the backward's binning plan (tests/bin_plan.py)
predicts the library's workspace size exactly (CPU only: the size is computed on
the host)."""
import ctypes

import pytest

import bin_plan

CASES = [(4, 8, 22223, 4, 4, 22223), (8, 8, 300, 4, 4, 22223), (1, 2, 256, 4, 32, 163),
         (1, 2, 100, 4, 32, 21760), (1, 1, 7000, 4, 16, 300), (2, 8, 43110, 4, 8, 43110),
         (1, 2, 16, 2, 2, 80), (3, 5, 37, 3, 3, 250), (1, 1, 1, 1, 1, 1), (2, 3, 0, 2, 2, 40),
         (5, 1, 4000, 1, 9, 1000)]


@pytest.mark.parametrize("case", CASES)
def test_plan_restatement_matches_library(case):
    import scale_deformable_attention_amd as msda
    from scale_deformable_attention_amd._binding import MsdaDims
    B, M, Nq, L, K, Nv = case
    n = ctypes.c_size_t()
    st = msda.library().msda_backward_workspace_size(ctypes.byref(MsdaDims(B, Nv, M, 32, L, Nq, K)),
                                                     0, ctypes.byref(n))
    assert st == 0
    assert n.value == bin_plan.workspace_bytes(B, M, Nq, L, K, Nv)
