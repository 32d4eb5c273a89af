"""The C-ABI library loads and exports what include/msda.h declares, and its
host-side argument checks reject bad calls before anything reaches a GPU.
Runs without a GPU: every call here returns before the first HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import scale_deformable_attention_amd as msda
from scale_deformable_attention_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["msda_backward", "msda_backward_ex", "msda_backward_fused",
                                    "msda_backward_fused_workspace_size", "msda_backward_noalloc",
                                    "msda_backward_workspace_min_size",
                                    "msda_backward_workspace_size", "msda_check_tables",
                                    "msda_dcn_backward", "msda_dcn_backward_workspace_size",
                                    "msda_dcn_forward", "msda_forward", "msda_forward_ex",
                                    "msda_forward_fused",
                                    "msda_layer_backward", "msda_layer_forward",
                                    "msda_layer_saved_size", "msda_layer_workspace_size",
                                    "msda_linear_backward",
                                    "msda_linear_backward_workspace_size",
                                    "msda_linear_forward", "msda_status_string",
                                    "msda_version"]


def test_library_exports_every_declared_symbol():
    lib = msda.library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported by libmsda.so"


def test_version_and_status_strings():
    lib = msda.library()
    assert lib.msda_version() == 700
    for s in range(5):
        assert len(lib.msda_status_string(s)) > 0
    assert lib.msda_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: checks return first


def fwd_status(dims, dtype=0, **ptrs):
    p = dict(value=FAKE, shapes=FAKE, lsi=FAKE, loc=FAKE, attn=FAKE, out=FAKE)
    p.update(ptrs)
    return msda.library().msda_forward(
        None if dims is None else ctypes.byref(dims), dtype, p["value"], p["shapes"], p["lsi"],
        p["loc"], p["attn"], p["out"], None)


def bwd_status(dims, dtype=0, ws_bytes=1 << 40, **ptrs):
    p = dict(value=FAKE, shapes=FAKE, lsi=FAKE, loc=FAKE, attn=FAKE, gout=FAKE, gv=FAKE,
             gl=FAKE, ga=FAKE, ws=FAKE)
    p.update(ptrs)
    return msda.library().msda_backward(
        None if dims is None else ctypes.byref(dims), dtype, p["value"], p["shapes"], p["lsi"],
        p["loc"], p["attn"], p["gout"], p["gv"], p["gl"], p["ga"], p["ws"],
        ctypes.c_size_t(ws_bytes), None)


def fused_fwd_status(dims, dtype=0, **ptrs):
    p = dict(value=FAKE, shapes=FAKE, lsi=FAKE, ref=FAKE, off=FAKE, logits=FAKE, out=FAKE)
    p.update(ptrs)
    return msda.library().msda_forward_fused(
        None if dims is None else ctypes.byref(dims), dtype, p["value"], p["shapes"], p["lsi"],
        p["ref"], p["off"], p["logits"], p["out"], None)


def fused_bwd_status(dims, dtype=0, ws_bytes=1 << 40, **ptrs):
    p = dict(value=FAKE, shapes=FAKE, lsi=FAKE, ref=FAKE, off=FAKE, logits=FAKE, gout=FAKE,
             gv=FAKE, gref=FAKE, goff=FAKE, glog=FAKE, ws=FAKE)
    p.update(ptrs)
    return msda.library().msda_backward_fused(
        None if dims is None else ctypes.byref(dims), dtype, p["value"], p["shapes"], p["lsi"],
        p["ref"], p["off"], p["logits"], p["gout"], p["gv"], p["gref"], p["goff"], p["glog"],
        p["ws"], ctypes.c_size_t(ws_bytes), None)


ALL_STATUS_FNS = [fwd_status, bwd_status, fused_fwd_status, fused_bwd_status]


def dims(**kw):
    d = dict(B=1, Nv=80, M=2, D=8, L=2, Nq=16, K=2)
    d.update(kw)
    return _binding.MsdaDims(*[d[k] for k in ("B", "Nv", "M", "D", "L", "Nq", "K")])


INVALID, UNSUPPORTED = 1, 2


@pytest.mark.parametrize("status_fn", ALL_STATUS_FNS)
def test_invalid_sizes(status_fn):
    assert status_fn(None) == INVALID
    for bad in (dict(B=-1), dict(Nq=-3), dict(K=-1), dict(M=0), dict(Nv=0), dict(L=0),
                dict(D=0)):
        assert status_fn(dims(**bad)) == INVALID, bad
    assert status_fn(dims(), dtype=7) == INVALID


@pytest.mark.parametrize("status_fn", ALL_STATUS_FNS)
def test_unsupported_sizes(status_fn):
    for d in (4, 12, 24, 128):
        assert status_fn(dims(D=d)) == UNSUPPORTED, d
    assert status_fn(dims(L=17, Nv=17)) == UNSUPPORTED
    # value tensor of 2 GiB or more
    assert status_fn(dims(B=4, Nv=2 ** 22, M=8, D=64)) == UNSUPPORTED
    # too many tuples for 32-bit indexing
    assert status_fn(dims(B=2 ** 12, Nq=2 ** 16, M=16)) == UNSUPPORTED


def test_null_and_misaligned_pointers():
    for key in ("value", "shapes", "lsi", "loc", "attn", "out"):
        assert fwd_status(dims(), **{key: None}) == INVALID, key
    for key in ("value", "shapes", "lsi", "loc", "attn", "gout"):
        assert bwd_status(dims(), **{key: None}) == INVALID, key
    odd = ctypes.c_void_p(0x10004)        # 4-byte but not 8/16-byte aligned
    for key in ("value", "out", "loc", "shapes", "lsi"):
        assert fwd_status(dims(), **{key: odd}) == INVALID, key
    for key in ("value", "gout", "gv", "loc", "gl"):
        assert bwd_status(dims(), **{key: odd}) == INVALID, key
    assert fwd_status(dims(), attn=ctypes.c_void_p(0x10002)) == INVALID


def test_fused_null_and_misaligned_pointers():
    for key in ("value", "shapes", "lsi", "ref", "off", "logits", "out"):
        assert fused_fwd_status(dims(), **{key: None}) == INVALID, key
    for key in ("value", "shapes", "lsi", "ref", "off", "logits", "gout"):
        assert fused_bwd_status(dims(), **{key: None}) == INVALID, key
    odd = ctypes.c_void_p(0x10004)
    for key in ("value", "out", "ref", "off", "shapes", "lsi"):
        assert fused_fwd_status(dims(), **{key: odd}) == INVALID, key
    for key in ("value", "gout", "gv", "ref", "off", "gref", "goff"):
        assert fused_bwd_status(dims(), **{key: odd}) == INVALID, key
    assert fused_fwd_status(dims(), logits=ctypes.c_void_p(0x10002)) == INVALID
    assert fused_bwd_status(dims(), glog=ctypes.c_void_p(0x10002)) == INVALID


def workspace_size(d, dtype=0):
    n = ctypes.c_size_t(0)
    st = msda.library().msda_backward_workspace_size(ctypes.byref(d), dtype, ctypes.byref(n))
    return st, n.value


def test_workspace_size_and_checks():
    st, n = workspace_size(dims())
    assert st == 0 and n > 0 and n % 256 == 0
    # grows with the point count, needs no level shapes
    st2, n2 = workspace_size(dims(Nq=1600))
    assert st2 == 0 and n2 > n
    assert workspace_size(dims(D=12))[0] == UNSUPPORTED
    assert msda.library().msda_backward_workspace_size(ctypes.byref(dims()), 0, None) == INVALID
    # a workspace smaller than one (b, m) plane's bins, missing or misaligned
    # is rejected before any launch (between one plane's and n bytes the value
    # gradient runs in several passes)
    import bin_plan
    one_plane = bin_plan.workspace_bytes(1, 2, 16, 2, 2, 80, planes=1)
    m = ctypes.c_size_t(0)
    assert msda.library().msda_backward_workspace_min_size(ctypes.byref(dims()), 0,
                                                           ctypes.byref(m)) == 0
    assert m.value == one_plane < n
    assert bwd_status(dims(), ws_bytes=one_plane - 1) == INVALID
    assert bwd_status(dims(), ws=None) == INVALID
    assert bwd_status(dims(), ws=ctypes.c_void_p(0x10010)) == INVALID
    # no grad_value: no workspace needed (the call then launches, so only the
    # argument check is exercised here with a bad dims to stop before it)
    assert bwd_status(dims(D=12), gv=None, ws=None, ws_bytes=0) == UNSUPPORTED


def test_fused_workspace_size_and_checks():
    n = ctypes.c_size_t(0)
    lib = msda.library()
    assert lib.msda_backward_fused_workspace_size(ctypes.byref(dims()), 0, ctypes.byref(n)) == 0
    core = workspace_size(dims())[1]
    # the fused plan adds the softmax statistics and an offset-gradient buffer
    assert n.value > core and n.value % 256 == 0
    assert lib.msda_backward_fused_workspace_size(ctypes.byref(dims(D=12)), 0,
                                                  ctypes.byref(n)) == UNSUPPORTED
    assert lib.msda_backward_fused_workspace_size(ctypes.byref(dims()), 0, None) == INVALID
    lib.msda_backward_fused_workspace_size(ctypes.byref(dims()), 0, ctypes.byref(n))
    # fixed part (softmax statistics, offset-gradient room) + one plane's bins
    import bin_plan
    fixed = n.value - core
    one_plane = fixed + bin_plan.workspace_bytes(1, 2, 16, 2, 2, 80, planes=1)
    assert fused_bwd_status(dims(), ws_bytes=one_plane - 1) == INVALID
    assert fused_bwd_status(dims(), ws=None) == INVALID
    assert fused_bwd_status(dims(), ws=ctypes.c_void_p(0x10010)) == INVALID


def test_check_tables():
    assert msda.msda_check_tables([[8, 8], [4, 4]], [0, 64], 80) == 0
    assert msda.msda_check_tables([[8, 8], [4, 4]], [0, 63], 80) == INVALID
    assert msda.msda_check_tables([[8, 8], [4, 4]], [0, 64], 81) == INVALID
    assert msda.msda_check_tables([[8, 0], [4, 4]], [0, 0], 16) == INVALID
    assert msda.msda_check_tables(np.zeros((17, 2), np.int64) + 1, np.arange(17), 17) == INVALID


def test_binding_rejects_cpu_tensors():
    import torch
    v = torch.zeros(1, 80, 2, 8)
    with pytest.raises(ValueError):
        msda.msda_forward(v, torch.zeros(2, 2, dtype=torch.int64), torch.zeros(2, dtype=torch.int64),
                          torch.zeros(1, 16, 2, 2, 2, 2), torch.zeros(1, 16, 2, 2, 2))
    with pytest.raises(ValueError):
        msda.msda_forward_fused(v, torch.zeros(2, 2, dtype=torch.int64),
                                torch.zeros(2, dtype=torch.int64), torch.zeros(1, 16, 2, 2),
                                torch.zeros(1, 16, 2, 2, 2, 2), torch.zeros(1, 16, 2, 4))


def test_linear_argument_checks():
    lib = msda.library()
    assert lib.msda_linear_forward(-1, 4, 4, FAKE, FAKE, None, FAKE, None) == INVALID
    assert lib.msda_linear_forward(4, 0, 4, FAKE, FAKE, None, FAKE, None) == INVALID
    assert lib.msda_linear_forward(4, 4, 4, None, FAKE, None, FAKE, None) == INVALID
    assert lib.msda_linear_forward(4, 4, 4, ctypes.c_void_p(0x10002), FAKE, None, FAKE,
                                   None) == INVALID
    assert lib.msda_linear_forward(1 << 30, 4, 4, FAKE, FAKE, None, FAKE, None) == UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert lib.msda_linear_backward_workspace_size(1000, 256, 256, ctypes.byref(n)) == 0
    assert n.value >= 256 * 256 * 4
    # weight gradient without (enough) workspace
    assert lib.msda_linear_backward(1000, 256, 256, FAKE, FAKE, FAKE, None, FAKE, None, None, 0,
                                    None) == INVALID
    assert lib.msda_linear_backward(1000, 256, 256, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                                    n.value - 1, None) == INVALID


def test_layer_sizes_and_checks():
    lib = msda.library()
    d = dims(M=2, D=8, K=2)
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.msda_layer_saved_size(ctypes.byref(d), ctypes.byref(a)) == 0
    assert lib.msda_layer_workspace_size(ctypes.byref(d), ctypes.byref(b)) == 0
    # saved: value [B,Nv,C], offsets, logits, core
    C, A = 16, 2 * 2 * 2
    assert a.value >= 4 * (80 * C + 16 * (2 * A) + 16 * A + 16 * C)
    assert b.value > 0 and a.value % 256 == 0 and b.value % 256 == 0
    assert lib.msda_layer_saved_size(ctypes.byref(dims(D=12)), ctypes.byref(a)) == UNSUPPORTED
    assert lib.msda_layer_saved_size(ctypes.byref(dims(K=0)), ctypes.byref(a)) == UNSUPPORTED
    assert lib.msda_layer_saved_size(None, ctypes.byref(a)) == INVALID
    params = _binding.MsdaLayerParams()
    for n in _binding.LAYER_PARAMS:
        setattr(params, n, 0x10000)
    lib.msda_layer_saved_size(ctypes.byref(d), ctypes.byref(a))
    args = (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(params), FAKE)
    # saved buffer missing, too small or misaligned
    assert lib.msda_layer_forward(*args, None, a.value, None) == INVALID
    assert lib.msda_layer_forward(*args, FAKE, a.value - 1, None) == INVALID
    assert lib.msda_layer_forward(*args, ctypes.c_void_p(0x10010), a.value, None) == INVALID
    # a weight missing
    params.attn_weight = None
    assert lib.msda_layer_forward(*args, FAKE, a.value, None) == INVALID


def dcn_dims(**kw):
    d = dict(B=1, H=6, W=7, G=2, D=8, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1, pad_h=1,
             pad_w=1, dilation_h=1, dilation_w=1, H_out=6, W_out=7)
    d.update(kw)
    return _binding.MsdaDcnDims(*[d[f] for f, _ in _binding.MsdaDcnDims._fields_])


def test_dcn_argument_checks():
    lib = msda.library()
    fwd = lambda d, **p: lib.msda_dcn_forward(  # noqa: E731
        None if d is None else ctypes.byref(d), 0, p.get("inp", FAKE), p.get("off", FAKE),
        p.get("mask", FAKE), p.get("out", FAKE), None)
    assert fwd(None) == INVALID
    for bad in (dict(H=0), dict(G=0), dict(kernel_w=0), dict(stride_h=0), dict(pad_w=-1),
                dict(dilation_h=0), dict(H_out=-1), dict(B=-1)):
        assert fwd(dcn_dims(**bad)) == INVALID, bad
    assert fwd(dcn_dims(D=12)) == UNSUPPORTED
    assert fwd(dcn_dims(W_out=1 << 24)) == UNSUPPORTED
    for key in ("inp", "off", "mask", "out"):
        assert fwd(dcn_dims(), **{key: None}) == INVALID, key
    assert fwd(dcn_dims(), off=ctypes.c_void_p(0x10004)) == INVALID
    n = ctypes.c_size_t(0)
    assert lib.msda_dcn_backward_workspace_size(ctypes.byref(dcn_dims()), 0, ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % 256 == 0
    bwd = lambda ws, nbytes: lib.msda_dcn_backward(  # noqa: E731
        ctypes.byref(dcn_dims()), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, ws,
        ctypes.c_size_t(nbytes), None)
    assert bwd(None, 0) == INVALID
    import bin_plan   # the grouped problem as a core one: 2 planes of 42 pixels, 9 points
    one_plane = bin_plan.workspace_bytes(1, 2, 42, 1, 9, 42, planes=1)
    assert one_plane < n.value
    assert bwd(FAKE, one_plane - 1) == INVALID


def test_precision_checks():
    lib = msda.library()
    P = _binding.MsdaPrecision
    fwd = lambda pr, **p: lib.msda_forward_ex(  # noqa: E731
        ctypes.byref(dims()), None if pr is None else ctypes.byref(pr), FAKE, FAKE, FAKE,
        p.get("loc", FAKE), p.get("attn", FAKE), FAKE, None)
    assert fwd(None) == INVALID
    assert fwd(P(3, 0, 0)) == INVALID          # unknown value type
    assert fwd(P(0, 1, 0)) == INVALID          # bf16 locations are not offered
    assert fwd(P(0, 0, 2)) == INVALID          # f16 grad_value is not offered
    # binary16 locations need 4-byte, weights 2-byte alignment only
    assert fwd(P(2, 2, 0), loc=ctypes.c_void_p(0x10002)) == INVALID
    assert fwd(P(0, 0, 0), loc=ctypes.c_void_p(0x10004)) == INVALID
    bwd = lambda pr, gv: lib.msda_backward_ex(  # noqa: E731
        ctypes.byref(dims()), ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gv, FAKE,
        FAKE, FAKE, ctypes.c_size_t(1 << 40), None)
    assert bwd(P(0, 0, 1), ctypes.c_void_p(0x10008)) == INVALID   # bf16 grad_value 16-byte


def test_c_client_builds_and_reports_version():
    # include/msda.h compiles as C99 with gcc, and a C program linked to the
    # library reads its version (no GPU call)
    import subprocess
    import abi_client
    binary = abi_client.BINARY if os.path.exists(abi_client.BINARY) else abi_client.build()
    r = subprocess.run([binary], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip()) == msda.msda_version()


def test_noalloc_backward_checks():
    """The allocation-free backward checks its arguments like msda_backward and
    refuses, before any HIP call, a problem one of whose (b, m) planes needs
    more binning workspace than its static scratch holds."""
    lib = msda.library()

    def call(d, grad_value=FAKE):
        return lib.msda_backward_noalloc(None if d is None else ctypes.byref(d), 0, FAKE, FAKE,
                                         FAKE, FAKE, FAKE, FAKE, grad_value, FAKE, FAKE, None)
    assert call(None) == INVALID
    assert call(dims(D=12)) == UNSUPPORTED
    # one (b, m) plane's bins beyond the scratch: refused (larger problems whose
    # planes fit run in passes)
    big = dims(B=1, M=1, D=32, L=4, K=4, Nq=100000, Nv=22223)
    import bin_plan
    assert bin_plan.workspace_bytes(1, 1, 100000, 4, 4, 22223, planes=1) > \
        _binding.NOALLOC_SCRATCH_BYTES
    assert call(big) == 4
    assert b"allocation-free" in lib.msda_status_string(4)
