"""CPU oracle of the multi-scale deformable attention core (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path never does.

The arithmetic lives in ``msda_oracle.c`` (plain C, double accumulation, single
thread); this module only marshals numpy arrays into it. See the header of
``msda_oracle.c`` for what is computed and which passages of the pages each
step follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_i64 = ctypes.c_int64
_pd = ctypes.POINTER(ctypes.c_double)
_pf = ctypes.POINTER(ctypes.c_float)
_pi = ctypes.POINTER(ctypes.c_int64)


def library(path=None):
    """Load the oracle shared library, building it first when it is absent or
    older than its source (the build leaves a digest of the source next to the
    library)."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not _build.is_current():
            _build.build()
        _LIB = _bind(ctypes.CDLL(_build.LIBRARY))
        # the library must report the version the source declares
        want = source_version()
        got = _LIB.msda_oracle_version()
        if got != want:
            raise RuntimeError(f"oracle library reports version {got}, its source {want}: "
                               "stale build")
    return _LIB


def source_version():
    """The version number msda_oracle.c declares (msda_oracle_version)."""
    import re
    with open(_build.SOURCE) as f:
        m = re.search(r"int msda_oracle_version\(void\) \{ return (\d+); \}", f.read())
    if not m:
        raise RuntimeError("msda_oracle_version not found in the oracle source")
    return int(m.group(1))


def _bind(lib):
    lib.msda_oracle_forward.restype = ctypes.c_int
    lib.msda_oracle_forward.argtypes = [_i64] * 7 + [_pd, _pi, _pi, _pf, _pd, _pd, _pd]
    lib.msda_oracle_backward.restype = ctypes.c_int
    lib.msda_oracle_backward.argtypes = [_i64] * 7 + [_pd, _pi, _pi, _pf, _pd, _pd, _pd, _pd,
                                                      _pd, _pd, _pd, _pd]
    lib.msda_oracle_version.restype = ctypes.c_int
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _prep(value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
    value = np.ascontiguousarray(value, dtype=np.float64)
    shapes = np.ascontiguousarray(spatial_shapes, dtype=np.int64).reshape(-1, 2)
    lsi = np.ascontiguousarray(level_start_index, dtype=np.int64).reshape(-1)
    loc = np.ascontiguousarray(sampling_locations, dtype=np.float32)
    attn = np.ascontiguousarray(attention_weights, dtype=np.float64)
    if value.ndim != 4 or loc.ndim != 6 or attn.ndim != 5:
        raise ValueError("value must be [B,Nv,M,D], locations [B,Nq,M,L,K,2], "
                         "weights [B,Nq,M,L,K]")
    B, Nv, M, D = value.shape
    Bq, Nq, Mq, L, K, two = loc.shape
    if (Bq, Mq, two) != (B, M, 2) or attn.shape != (B, Nq, M, L, K):
        raise ValueError("inconsistent shapes")
    if shapes.shape[0] != L or lsi.shape[0] != L:
        raise ValueError("spatial_shapes / level_start_index do not have L rows")
    dims = (B, Nv, M, D, L, Nq, K)
    return dims, value, shapes, lsi, loc, attn


def forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            with_abs=False, lib=None):
    """Core forward in double. Returns out [B,Nq,M,D] (and the per-element
    absolute term sums when ``with_abs``). ``lib`` selects another build of
    the oracle (the default is the in-tree one)."""
    dims, value, shapes, lsi, loc, attn = _prep(value, spatial_shapes, level_start_index,
                                                sampling_locations, attention_weights)
    B, Nv, M, D, L, Nq, K = dims
    out = np.empty((B, Nq, M, D), np.float64)
    out_abs = np.empty_like(out) if with_abs else None
    rc = (lib or library()).msda_oracle_forward(*dims, _ptr(value, ctypes.c_double),
                                       _ptr(shapes, ctypes.c_int64), _ptr(lsi, ctypes.c_int64),
                                       _ptr(loc, ctypes.c_float), _ptr(attn, ctypes.c_double),
                                       _ptr(out, ctypes.c_double),
                                       _ptr(out_abs, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (tables inconsistent with Nv?)")
    return (out, out_abs) if with_abs else out


def backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
             grad_output, with_abs=False, lib=None):
    """Core backward in double. Returns (grad_value, grad_locations,
    grad_weights), followed by their absolute term sums when ``with_abs``."""
    dims, value, shapes, lsi, loc, attn = _prep(value, spatial_shapes, level_start_index,
                                                sampling_locations, attention_weights)
    B, Nv, M, D, L, Nq, K = dims
    g = np.ascontiguousarray(grad_output, dtype=np.float64).reshape(B, Nq, M, D)
    gv = np.empty((B, Nv, M, D), np.float64)
    gl = np.empty((B, Nq, M, L, K, 2), np.float64)
    ga = np.empty((B, Nq, M, L, K), np.float64)
    gva = np.empty_like(gv) if with_abs else None
    gla = np.empty_like(gl) if with_abs else None
    gaa = np.empty_like(ga) if with_abs else None
    rc = (lib or library()).msda_oracle_backward(*dims, _ptr(value, ctypes.c_double),
                                        _ptr(shapes, ctypes.c_int64), _ptr(lsi, ctypes.c_int64),
                                        _ptr(loc, ctypes.c_float), _ptr(attn, ctypes.c_double),
                                        _ptr(g, ctypes.c_double), _ptr(gv, ctypes.c_double),
                                        _ptr(gl, ctypes.c_double), _ptr(ga, ctypes.c_double),
                                        _ptr(gva, ctypes.c_double), _ptr(gla, ctypes.c_double),
                                        _ptr(gaa, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (tables inconsistent with Nv?)")
    if with_abs:
        return gv, gl, ga, gva, gla, gaa
    return gv, gl, ga


def _bind_fused(lib):
    if getattr(lib, "_fused_bound", False):
        return lib
    lib.msda_oracle_forward_fused.restype = ctypes.c_int
    lib.msda_oracle_forward_fused.argtypes = [_i64] * 7 + [_pd, _pi, _pi, _pf, _pf, _pf, _pd, _pd]
    lib.msda_oracle_backward_fused.restype = ctypes.c_int
    lib.msda_oracle_backward_fused.argtypes = [_i64] * 7 + [_pd, _pi, _pi, _pf, _pf, _pf, _pd] + \
        [_pd] * 8
    lib._fused_bound = True
    return lib


def _prep_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                attention_logits):
    value = np.ascontiguousarray(value, dtype=np.float64)
    shapes = np.ascontiguousarray(spatial_shapes, dtype=np.int64).reshape(-1, 2)
    lsi = np.ascontiguousarray(level_start_index, dtype=np.int64).reshape(-1)
    ref = np.ascontiguousarray(reference_points, dtype=np.float32)
    off = np.ascontiguousarray(sampling_offsets, dtype=np.float32)
    B, Nv, M, D = value.shape
    if off.ndim != 6 or off.shape[0] != B or off.shape[2] != M or off.shape[5] != 2:
        raise ValueError("offsets must be [B,Nq,M,L,K,2]")
    _, Nq, _, L, K, _ = off.shape
    logits = np.ascontiguousarray(attention_logits, dtype=np.float32).reshape(B, Nq, M, L * K)
    if ref.shape != (B, Nq, L, 2):
        raise ValueError("reference points must be [B,Nq,L,2]")
    if shapes.shape[0] != L or lsi.shape[0] != L:
        raise ValueError("spatial_shapes / level_start_index do not have L rows")
    return (B, Nv, M, D, L, Nq, K), value, shapes, lsi, ref, off, logits


def forward_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                  attention_logits, with_abs=False, lib=None):
    """Fused front-end + core forward in double: locations from reference
    points [B,Nq,L,2] and offsets [B,Nq,M,L,K,2] (level pixels), weights as the
    softmax of logits [B,Nq,M,L*K]. Returns out [B,Nq,M,D] (and the absolute
    term sums when ``with_abs``)."""
    dims, value, shapes, lsi, ref, off, logits = _prep_fused(
        value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
        attention_logits)
    B, Nv, M, D, L, Nq, K = dims
    out = np.empty((B, Nq, M, D), np.float64)
    out_abs = np.empty_like(out) if with_abs else None
    rc = _bind_fused(lib or library()).msda_oracle_forward_fused(
        *dims, _ptr(value, ctypes.c_double), _ptr(shapes, ctypes.c_int64),
        _ptr(lsi, ctypes.c_int64), _ptr(ref, ctypes.c_float), _ptr(off, ctypes.c_float),
        _ptr(logits, ctypes.c_float), _ptr(out, ctypes.c_double), _ptr(out_abs, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return (out, out_abs) if with_abs else out


def backward_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                   attention_logits, grad_output, with_abs=False, lib=None):
    """Fused backward in double. Returns (grad_value, grad_reference_points,
    grad_offsets, grad_logits), followed by their absolute term sums when
    ``with_abs``."""
    dims, value, shapes, lsi, ref, off, logits = _prep_fused(
        value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
        attention_logits)
    B, Nv, M, D, L, Nq, K = dims
    g = np.ascontiguousarray(grad_output, dtype=np.float64).reshape(B, Nq, M, D)
    outs = [np.empty((B, Nv, M, D)), np.empty((B, Nq, L, 2)), np.empty((B, Nq, M, L, K, 2)),
            np.empty((B, Nq, M, L * K))]
    abss = [np.empty_like(o) for o in outs] if with_abs else [None] * 4
    rc = _bind_fused(lib or library()).msda_oracle_backward_fused(
        *dims, _ptr(value, ctypes.c_double), _ptr(shapes, ctypes.c_int64),
        _ptr(lsi, ctypes.c_int64), _ptr(ref, ctypes.c_float), _ptr(off, ctypes.c_float),
        _ptr(logits, ctypes.c_float), _ptr(g, ctypes.c_double),
        *[_ptr(o, ctypes.c_double) for o in outs], *[_ptr(a, ctypes.c_double) for a in abss])
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return tuple(outs) + (tuple(abss) if with_abs else ())


# ----------------------------------------------------------------------------- DCNv3
def _bind_dcn(lib):
    if getattr(lib, "_dcn_bound", False):
        return lib
    lib.msda_oracle_dcn_forward.restype = ctypes.c_int
    lib.msda_oracle_dcn_forward.argtypes = [_i64] * 15 + [_pd, _pf, _pd, _pd, _pd]
    lib.msda_oracle_dcn_backward.restype = ctypes.c_int
    lib.msda_oracle_dcn_backward.argtypes = [_i64] * 15 + [_pd, _pf, _pd, _pd] + [_pd] * 6
    lib._dcn_bound = True
    return lib


def _prep_dcn(inp, offset, mask, kernel, stride, pad, dilation):
    inp = np.ascontiguousarray(inp, dtype=np.float64)
    off = np.ascontiguousarray(offset, dtype=np.float32)
    m = np.ascontiguousarray(mask, dtype=np.float64)
    B, H, W, G, D = inp.shape
    kh, kw = kernel
    if off.ndim != 6 or off.shape[0] != B or off.shape[3] != G or off.shape[4] != kh * kw \
            or off.shape[5] != 2:
        raise ValueError("offset must be [B, H_out, W_out, G, K, 2]")
    Ho, Wo = off.shape[1], off.shape[2]
    if m.shape != off.shape[:5]:
        raise ValueError("mask must be [B, H_out, W_out, G, K]")
    dims = (B, H, W, G, D, kh, kw, stride[0], stride[1], pad[0], pad[1], dilation[0],
            dilation[1], Ho, Wo)
    return dims, inp, off, m


def dcn_forward(inp, offset, mask, kernel, stride=(1, 1), pad=(0, 0), dilation=(1, 1),
                with_abs=False, lib=None):
    """DCNv3 aggregation in double (see msda_oracle.c): input [B,H,W,G,D],
    offset [B,Ho,Wo,G,K,2] pixels (x, y), mask [B,Ho,Wo,G,K] -> out
    [B,Ho,Wo,G,D] (and the absolute term sums with ``with_abs``)."""
    dims, inp, off, m = _prep_dcn(inp, offset, mask, kernel, stride, pad, dilation)
    B, H, W, G, D = inp.shape
    Ho, Wo = dims[13], dims[14]
    out = np.empty((B, Ho, Wo, G, D))
    out_abs = np.empty_like(out) if with_abs else None
    rc = _bind_dcn(lib or library()).msda_oracle_dcn_forward(
        *dims, _ptr(inp, ctypes.c_double), _ptr(off, ctypes.c_float), _ptr(m, ctypes.c_double),
        _ptr(out, ctypes.c_double), _ptr(out_abs, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return (out, out_abs) if with_abs else out


def dcn_backward(inp, offset, mask, grad_output, kernel, stride=(1, 1), pad=(0, 0),
                 dilation=(1, 1), with_abs=False, lib=None):
    """Gradients of dcn_forward: (grad_input, grad_offset, grad_mask), then
    their absolute term sums with ``with_abs``."""
    dims, inp, off, m = _prep_dcn(inp, offset, mask, kernel, stride, pad, dilation)
    B, H, W, G, D = inp.shape
    Ho, Wo = dims[13], dims[14]
    g = np.ascontiguousarray(grad_output, dtype=np.float64).reshape(B, Ho, Wo, G, D)
    outs = [np.empty(inp.shape), np.empty(off.shape), np.empty(m.shape)]
    abss = [np.empty_like(o) for o in outs] if with_abs else [None] * 3
    rc = _bind_dcn(lib or library()).msda_oracle_dcn_backward(
        *dims, _ptr(inp, ctypes.c_double), _ptr(off, ctypes.c_float), _ptr(m, ctypes.c_double),
        _ptr(g, ctypes.c_double), *[_ptr(o, ctypes.c_double) for o in outs],
        *[_ptr(a, ctypes.c_double) for a in abss])
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return tuple(outs) + (tuple(abss) if with_abs else ())
