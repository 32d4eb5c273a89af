"""bench.py names the forward kernel the library launches (the roofline and
the counter summaries refer to it by name). Its rule restates the library's
choice; this CPU test holds the two to the same constants and checks the
rule's decisions on the named workloads."""
import os
import re

import bench
from scale_deformable_attention_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "scale_deformable_attention_amd", "csrc", "msda.hip")


def _constant(text, name):
    m = re.search(r"constexpr int %s = ([0-9 *]+);" % name, text)
    assert m, name
    value = 1
    for factor in m.group(1).split("*"):
        value *= int(factor)
    return value


def test_constants_match_the_library():
    text = open(SOURCE).read()
    assert bench.STAGE_BYTES == _constant(text, "kStageBytes")
    assert bench.STAGED_MIN_QUERIES == _constant(text, "kStagedMinQueries")
    # the row widths with staged kernels
    assert "return row_bytes == 64 || row_bytes == 128;" in text


def test_decisions_on_the_named_workloads():
    w = wl.WORKLOADS
    # 800x1333 pyramid: coarsest level 13 x 21, estimated 261 pixels
    assert bench.forward_kernel(w["encoder_train"], 4) == "msda_fwd_staged_kernel"
    assert bench.forward_kernel(w["encoder"], 4) == "msda_fwd_staged_kernel"
    assert bench.forward_kernel(w["encoder_train"], 4, fused=True) == "msda_fwd_staged_kernel<fused>"
    # 1920x1080 pyramid at 64-byte bf16 rows: 505 estimated pixels fit 36 KB
    assert bench.forward_kernel(w["hires_bf16"], 2) == "msda_fwd_staged_kernel"
    # ... but not at 128-byte fp32 rows
    assert bench.forward_kernel(w["hires_bf16"], 4) == "msda_fwd_kernel"
    # 300 queries: plain
    assert bench.forward_kernel(w["decoder"], 4) == "msda_fwd_kernel"
    assert bench.forward_kernel(w["tiny"], 4) == "msda_fwd_kernel"
    # 256-byte rows (D = 64 fp32) have no staged kernel
    assert bench.forward_kernel(w["encoder_train"].scaled(D=64), 4) == "msda_fwd_kernel"
