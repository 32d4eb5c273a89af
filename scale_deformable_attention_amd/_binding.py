"""ctypes binding of libmsda.so (include/msda.h): argument marshalling only.

Every step of the core runs in the library's HIP kernels; this module checks
tensor shapes, dtypes and devices, allocates outputs with torch (device memory
is torch's), passes raw device pointers and the current HIP stream, and turns
a non-zero status into an exception. There is no fallback path: without the
built library every call raises.
"""
import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsda.so")

MSDA_DTYPE_F32 = 0
MSDA_DTYPE_BF16 = 1
MSDA_DTYPE_F16 = 2
STATUS = {0: "MSDA_SUCCESS", 1: "MSDA_ERROR_INVALID_VALUE", 2: "MSDA_ERROR_NOT_SUPPORTED",
          3: "MSDA_ERROR_LAUNCH", 4: "MSDA_ERROR_SCRATCH_TOO_SMALL"}
# scratch the allocation-free backward holds per GPU (include/msda.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


class MsdaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "Nv", "M", "D", "L", "Nq", "K")]


LAYER_PARAMS = ("value_weight", "value_bias", "offset_weight", "offset_bias", "attn_weight",
                "attn_bias", "output_weight", "output_bias")


class MsdaLayerParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_PARAMS]


class MsdaLayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_PARAMS]


class MsdaPrecision(ctypes.Structure):
    _fields_ = [("value", ctypes.c_int), ("locations", ctypes.c_int), ("grad_value", ctypes.c_int)]


class MsdaDcnDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("B", "H", "W", "G", "D", "kernel_h", "kernel_w", "stride_h", "stride_w", "pad_h",
                 "pad_w", "dilation_h", "dilation_w", "H_out", "W_out")]


class MsdaError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({library().msda_status_string(status).decode()})")
        self.status = status


_LIB = None


def library():
    """Load libmsda.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIBRARY)
        vp, i64p, fp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.msda_forward.restype = ctypes.c_int
        lib.msda_forward.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int, vp, i64p, i64p, fp,
                                     fp, fp, vp]
        lib.msda_backward.restype = ctypes.c_int
        lib.msda_backward.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int, vp, i64p, i64p, fp,
                                      fp, fp, fp, fp, fp, vp, ctypes.c_size_t, vp]
        lib.msda_backward_noalloc.restype = ctypes.c_int
        lib.msda_backward_noalloc.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int, vp, i64p,
                                              i64p, fp, fp, fp, fp, fp, fp, vp]
        lib.msda_backward_workspace_min_size.restype = ctypes.c_int
        lib.msda_backward_workspace_min_size.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int,
                                                         ctypes.POINTER(ctypes.c_size_t)]
        lib.msda_backward_workspace_size.restype = ctypes.c_int
        lib.msda_backward_workspace_size.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.msda_check_tables.restype = ctypes.c_int
        lib.msda_check_tables.argtypes = [i64p, i64p, ctypes.c_int64, ctypes.c_int64]
        lib.msda_status_string.restype = ctypes.c_char_p
        lib.msda_status_string.argtypes = [ctypes.c_int]
        lib.msda_version.restype = ctypes.c_int
        lib.msda_version.argtypes = []
        lib.msda_forward_fused.restype = ctypes.c_int
        lib.msda_forward_fused.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int, vp, i64p, i64p,
                                           fp, fp, fp, fp, vp]
        lib.msda_backward_fused.restype = ctypes.c_int
        lib.msda_backward_fused.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int, vp, i64p,
                                            i64p, fp, fp, fp, fp, fp, fp, fp, fp, vp,
                                            ctypes.c_size_t, vp]
        i64 = ctypes.c_int64
        lib.msda_linear_forward.restype = ctypes.c_int
        lib.msda_linear_forward.argtypes = [i64, i64, i64, fp, fp, fp, fp, vp]
        lib.msda_linear_backward.restype = ctypes.c_int
        lib.msda_linear_backward.argtypes = [i64, i64, i64, fp, fp, fp, fp, fp, fp, vp,
                                             ctypes.c_size_t, vp]
        lib.msda_linear_backward_workspace_size.restype = ctypes.c_int
        lib.msda_linear_backward_workspace_size.argtypes = [i64, i64, i64,
                                                            ctypes.POINTER(ctypes.c_size_t)]
        lp, lg = ctypes.POINTER(MsdaLayerParams), ctypes.POINTER(MsdaLayerGrads)
        lib.msda_layer_forward.restype = ctypes.c_int
        lib.msda_layer_forward.argtypes = [ctypes.POINTER(MsdaDims), fp, fp, fp, i64p, i64p, lp,
                                           fp, vp, ctypes.c_size_t, vp]
        lib.msda_layer_backward.restype = ctypes.c_int
        lib.msda_layer_backward.argtypes = [ctypes.POINTER(MsdaDims), fp, fp, fp, i64p, i64p, lp,
                                            vp, ctypes.c_size_t, fp, fp, fp, fp, lg, vp,
                                            ctypes.c_size_t, vp]
        for name in ("msda_layer_saved_size", "msda_layer_workspace_size"):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [ctypes.POINTER(MsdaDims),
                                           ctypes.POINTER(ctypes.c_size_t)]
        dp = ctypes.POINTER(MsdaDcnDims)
        lib.msda_dcn_forward.restype = ctypes.c_int
        lib.msda_dcn_forward.argtypes = [dp, ctypes.c_int, vp, fp, fp, fp, vp]
        lib.msda_dcn_backward.restype = ctypes.c_int
        lib.msda_dcn_backward.argtypes = [dp, ctypes.c_int, vp, fp, fp, fp, fp, fp, fp, vp,
                                          ctypes.c_size_t, vp]
        lib.msda_dcn_backward_workspace_size.restype = ctypes.c_int
        lib.msda_dcn_backward_workspace_size.argtypes = [dp, ctypes.c_int,
                                                         ctypes.POINTER(ctypes.c_size_t)]
        pp = ctypes.POINTER(MsdaPrecision)
        lib.msda_forward_ex.restype = ctypes.c_int
        lib.msda_forward_ex.argtypes = [ctypes.POINTER(MsdaDims), pp, vp, i64p, i64p, vp, vp, fp,
                                        vp]
        lib.msda_backward_ex.restype = ctypes.c_int
        lib.msda_backward_ex.argtypes = [ctypes.POINTER(MsdaDims), pp, vp, i64p, i64p, vp, vp, fp,
                                         vp, fp, fp, vp, ctypes.c_size_t, vp]
        lib.msda_backward_fused_workspace_size.restype = ctypes.c_int
        lib.msda_backward_fused_workspace_size.argtypes = [ctypes.POINTER(MsdaDims), ctypes.c_int,
                                                           ctypes.POINTER(ctypes.c_size_t)]
        _LIB = lib
    return _LIB


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dims(value, spatial_shapes, sampling_locations, attention_weights):
    if value.dim() != 4:
        raise ValueError("value must be [B, Nv, M, D]")
    if sampling_locations.dim() != 6 or sampling_locations.shape[-1] != 2:
        raise ValueError("sampling_locations must be [B, Nq, M, L, K, 2]")
    B, Nv, M, D = value.shape
    Bq, Nq, Mq, L, K, _ = sampling_locations.shape
    if (Bq, Mq) != (B, M):
        raise ValueError("sampling_locations batch/head sizes differ from value's")
    if tuple(attention_weights.shape) != (B, Nq, M, L, K):
        raise ValueError("attention_weights must be [B, Nq, M, L, K]")
    if tuple(spatial_shapes.shape) != (L, 2):
        raise ValueError("spatial_shapes must be [L, 2]")
    return MsdaDims(B, Nv, M, D, L, Nq, K)


def _check(t, name, dtypes, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


VALUE_DTYPES = (torch.float32, torch.bfloat16, torch.float16)


def _value_dtype(value):
    if value.dtype == torch.float32:
        return MSDA_DTYPE_F32
    if value.dtype == torch.bfloat16:
        return MSDA_DTYPE_BF16
    if value.dtype == torch.float16:
        return MSDA_DTYPE_F16
    raise ValueError(f"value dtype {value.dtype} is not supported (float32, bfloat16, float16)")


def _precision(value, sampling_locations, grad_value_dtype=torch.float32):
    return MsdaPrecision(_value_dtype(value),
                         MSDA_DTYPE_F16 if sampling_locations.dtype == torch.float16
                         else MSDA_DTYPE_F32,
                         MSDA_DTYPE_BF16 if grad_value_dtype == torch.bfloat16 else MSDA_DTYPE_F32)


def _common(value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
    dev = value.device
    if dev.type != "cuda":
        raise ValueError("value must be a GPU tensor")
    _check(value, "value", VALUE_DTYPES, dev)
    _check(spatial_shapes, "spatial_shapes", (torch.int64,), dev)
    _check(level_start_index, "level_start_index", (torch.int64,), dev)
    _check(sampling_locations, "sampling_locations", (torch.float32, torch.float16), dev)
    _check(attention_weights, "attention_weights", (sampling_locations.dtype,), dev)
    dims = _dims(value, spatial_shapes, sampling_locations, attention_weights)
    if tuple(level_start_index.shape) != (dims.L,):
        raise ValueError("level_start_index must be [L]")
    return dev, dims


def msda_forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                 output=None, stream=None):
    """Core forward (include/msda.h msda_forward). Returns output [B, Nq, M*D]
    (fp32); ``output`` may be passed to write into an existing tensor."""
    dev, dims = _common(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights)
    if output is None:
        output = torch.empty((dims.B, dims.Nq, dims.M * dims.D), dtype=torch.float32, device=dev)
    else:
        _check(output, "output", (torch.float32,), dev)
        if output.numel() != dims.B * dims.Nq * dims.M * dims.D:
            raise ValueError("output has the wrong number of elements")
    pr = _precision(value, sampling_locations)
    st = library().msda_forward_ex(ctypes.byref(dims), ctypes.byref(pr), _ptr(value),
                                   _ptr(spatial_shapes), _ptr(level_start_index),
                                   _ptr(sampling_locations), _ptr(attention_weights), _ptr(output),
                                   _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_forward")
    return output


def msda_backward_workspace_min_size(value, sampling_locations):
    """Smallest workspace msda_backward accepts for these tensors' sizes (the
    value gradient then runs one (b, m) plane per pass)."""
    B, Nv, M, Dv = value.shape
    _, Nq, _, L, K, _ = sampling_locations.shape
    dims = MsdaDims(B, Nv, M, Dv, L, Nq, K)
    n = ctypes.c_size_t(0)
    st = library().msda_backward_workspace_min_size(ctypes.byref(dims), _value_dtype(value),
                                                    ctypes.byref(n))
    if st != 0:
        raise MsdaError(st, "msda_backward_workspace_min_size")
    return n.value


def msda_backward_workspace_size(value, sampling_locations, D=None):
    """Workspace bytes msda_backward needs for these tensors' sizes."""
    B, Nv, M, Dv = value.shape
    _, Nq, _, L, K, _ = sampling_locations.shape
    dims = MsdaDims(B, Nv, M, Dv, L, Nq, K)
    n = ctypes.c_size_t(0)
    st = library().msda_backward_workspace_size(ctypes.byref(dims), _value_dtype(value),
                                                ctypes.byref(n))
    if st != 0:
        raise MsdaError(st, "msda_backward_workspace_size")
    return n.value


def msda_backward_noalloc(value, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, grad_output, grad_value=None,
                          grad_sampling_locations=None, grad_attention_weights=None,
                          needs=(True, True, True), stream=None):
    """Core backward through msda_backward_noalloc (include/msda.h): no
    workspace; the library's static per-GPU scratch serves instead. fp32
    gradients, value fp32, bf16 or f16. Returns (grad_value,
    grad_sampling_locations, grad_attention_weights) like msda_backward; the
    gradients not given are allocated here (by torch), the call itself
    allocates nothing. Raises MsdaError (MSDA_ERROR_SCRATCH_TOO_SMALL) for a
    problem whose binning workspace exceeds the static scratch."""
    dev, dims = _common(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights)
    if sampling_locations.dtype != torch.float32 or attention_weights.dtype != torch.float32:
        raise ValueError("msda_backward_noalloc takes fp32 locations and weights")
    _check(grad_output, "grad_output", (torch.float32,), dev)
    if grad_output.numel() != dims.B * dims.Nq * dims.M * dims.D:
        raise ValueError("grad_output has the wrong number of elements")
    outs = []
    for need, given, shape, name in (
            (needs[0], grad_value, (dims.B, dims.Nv, dims.M, dims.D), "grad_value"),
            (needs[1], grad_sampling_locations, tuple(sampling_locations.shape),
             "grad_sampling_locations"),
            (needs[2], grad_attention_weights, tuple(attention_weights.shape),
             "grad_attention_weights")):
        if not need:
            outs.append(None)
        elif given is None:
            outs.append(torch.empty(shape, dtype=torch.float32, device=dev))
        else:
            _check(given, name, (torch.float32,), dev)
            if tuple(given.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
            outs.append(given)
    st = library().msda_backward_noalloc(ctypes.byref(dims), _value_dtype(value), _ptr(value),
                                         _ptr(spatial_shapes), _ptr(level_start_index),
                                         _ptr(sampling_locations), _ptr(attention_weights),
                                         _ptr(grad_output), _ptr(outs[0]), _ptr(outs[1]),
                                         _ptr(outs[2]), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_backward_noalloc")
    return tuple(outs)


def msda_backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                  grad_output, grad_value=None, grad_sampling_locations=None,
                  grad_attention_weights=None, needs=(True, True, True), workspace=None,
                  stream=None, grad_value_dtype=torch.float32):
    """Core backward (include/msda.h msda_backward / msda_backward_ex).
    Returns (grad_value, grad_sampling_locations, grad_attention_weights);
    the location and weight gradients are fp32, grad_value is fp32 or, with
    ``grad_value_dtype=torch.bfloat16``, bf16. An entry of ``needs`` set to
    False skips (and returns None for) that gradient. ``workspace`` (a uint8
    GPU tensor; msda_backward_workspace_size bytes run the value gradient in
    one pass, fewer -- down to one (b, m) plane's bins -- in several) is
    allocated here when not given and grad_value is needed."""
    dev, dims = _common(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights)
    _check(grad_output, "grad_output", (torch.float32,), dev)
    if grad_output.numel() != dims.B * dims.Nq * dims.M * dims.D:
        raise ValueError("grad_output has the wrong number of elements")
    if grad_value_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_value_dtype must be float32 or bfloat16")
    outs = []
    for need, given, shape, name, dt in (
            (needs[0], grad_value, (dims.B, dims.Nv, dims.M, dims.D), "grad_value",
             grad_value_dtype),
            (needs[1], grad_sampling_locations, tuple(sampling_locations.shape),
             "grad_sampling_locations", torch.float32),
            (needs[2], grad_attention_weights, tuple(attention_weights.shape),
             "grad_attention_weights", torch.float32)):
        if not need:
            outs.append(None)
        elif given is None:
            outs.append(torch.empty(shape, dtype=dt, device=dev))
        else:
            _check(given, name, (dt,), dev)
            if tuple(given.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
            outs.append(given)
    ws_bytes = 0
    if outs[0] is not None:
        n = ctypes.c_size_t(0)
        st = library().msda_backward_workspace_size(ctypes.byref(dims), _value_dtype(value),
                                                    ctypes.byref(n))
        if st != 0:
            raise MsdaError(st, "msda_backward_workspace_size")
        if workspace is None:
            workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
        elif workspace.device != dev or workspace.dtype != torch.uint8:
            # a smaller workspace than msda_backward_workspace_size is used in
            # several passes over the (b, m) planes; the library refuses one
            # that does not hold a single plane's bins
            raise ValueError(f"workspace must be a uint8 tensor on {dev}")
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    pr = _precision(value, sampling_locations, grad_value_dtype)
    st = library().msda_backward_ex(ctypes.byref(dims), ctypes.byref(pr), _ptr(value),
                                    _ptr(spatial_shapes), _ptr(level_start_index),
                                    _ptr(sampling_locations), _ptr(attention_weights),
                                    _ptr(grad_output), _ptr(outs[0]), _ptr(outs[1]),
                                    _ptr(outs[2]), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                                    _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_backward")
    return tuple(outs)


def msda_check_tables(spatial_shapes, level_start_index, Nv):
    """Host check of the level tables (include/msda.h msda_check_tables)."""
    import numpy as np
    s = np.ascontiguousarray(np.asarray(spatial_shapes, np.int64).reshape(-1, 2))
    i = np.ascontiguousarray(np.asarray(level_start_index, np.int64).reshape(-1))
    return library().msda_check_tables(s.ctypes.data, i.ctypes.data, s.shape[0], int(Nv))


def msda_version():
    return library().msda_version()


class MSDeformAttnFunction(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in the HIP library."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights):
        ctx.save_for_backward(value, spatial_shapes, level_start_index, sampling_locations,
                              attention_weights)
        return msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights)

    @staticmethod
    def backward(ctx, grad_output):
        value, shapes, lsi, loc, attn = ctx.saved_tensors
        needs = (ctx.needs_input_grad[0], ctx.needs_input_grad[3], ctx.needs_input_grad[4])
        # a bf16 value takes its gradient as bf16 straight from the kernel
        gdt = torch.bfloat16 if value.dtype == torch.bfloat16 else torch.float32
        gv, gl, ga = msda_backward(value, shapes, lsi, loc, attn, grad_output.contiguous(),
                                   needs=needs, grad_value_dtype=gdt)
        if gv is not None and gv.dtype != value.dtype:
            gv = gv.to(value.dtype)
        if gl is not None and gl.dtype != loc.dtype:
            gl = gl.to(loc.dtype)
        if ga is not None and ga.dtype != attn.dtype:
            ga = ga.to(attn.dtype)
        return gv, None, None, gl, ga


def ms_deform_attn(value, spatial_shapes, level_start_index, sampling_locations,
                   attention_weights):
    """Differentiable core: output [B, Nq, M*D]."""
    return MSDeformAttnFunction.apply(value, spatial_shapes, level_start_index,
                                      sampling_locations, attention_weights)


# ----------------------------------------------------------------------------- fused front-end
def _common_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                  attention_logits):
    dev = value.device
    if dev.type != "cuda":
        raise ValueError("value must be a GPU tensor")
    _check(value, "value", VALUE_DTYPES, dev)
    _check(spatial_shapes, "spatial_shapes", (torch.int64,), dev)
    _check(level_start_index, "level_start_index", (torch.int64,), dev)
    _check(reference_points, "reference_points", (torch.float32,), dev)
    _check(sampling_offsets, "sampling_offsets", (torch.float32,), dev)
    _check(attention_logits, "attention_logits", (torch.float32,), dev)
    if value.dim() != 4:
        raise ValueError("value must be [B, Nv, M, D]")
    if sampling_offsets.dim() != 6 or sampling_offsets.shape[-1] != 2:
        raise ValueError("sampling_offsets must be [B, Nq, M, L, K, 2]")
    B, Nv, M, D = value.shape
    Bq, Nq, Mq, L, K, _ = sampling_offsets.shape
    if (Bq, Mq) != (B, M):
        raise ValueError("sampling_offsets batch/head sizes differ from value's")
    if tuple(reference_points.shape) != (B, Nq, L, 2):
        raise ValueError("reference_points must be [B, Nq, L, 2]")
    if tuple(attention_logits.shape) not in ((B, Nq, M, L * K), (B, Nq, M, L, K)):
        raise ValueError("attention_logits must be [B, Nq, M, L*K]")
    if tuple(spatial_shapes.shape) != (L, 2) or tuple(level_start_index.shape) != (L,):
        raise ValueError("spatial_shapes must be [L, 2] and level_start_index [L]")
    return dev, MsdaDims(B, Nv, M, D, L, Nq, K)


def msda_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                       sampling_offsets, attention_logits, output=None, stream=None):
    """Fused forward (include/msda.h msda_forward_fused): locations from the
    reference points [B,Nq,L,2] and offsets [B,Nq,M,L,K,2] (level pixels),
    weights as the softmax of the logits [B,Nq,M,L*K], both formed in the
    kernel. Returns output [B, Nq, M*D] (fp32)."""
    dev, dims = _common_fused(value, spatial_shapes, level_start_index, reference_points,
                              sampling_offsets, attention_logits)
    if output is None:
        output = torch.empty((dims.B, dims.Nq, dims.M * dims.D), dtype=torch.float32, device=dev)
    else:
        _check(output, "output", (torch.float32,), dev)
        if output.numel() != dims.B * dims.Nq * dims.M * dims.D:
            raise ValueError("output has the wrong number of elements")
    st = library().msda_forward_fused(ctypes.byref(dims), _value_dtype(value), _ptr(value),
                                      _ptr(spatial_shapes), _ptr(level_start_index),
                                      _ptr(reference_points), _ptr(sampling_offsets),
                                      _ptr(attention_logits), _ptr(output), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_forward_fused")
    return output


def msda_backward_fused_workspace_size(value, sampling_offsets):
    """Workspace bytes msda_backward_fused needs for these tensors' sizes."""
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = sampling_offsets.shape
    dims = MsdaDims(B, Nv, M, D, L, Nq, K)
    n = ctypes.c_size_t(0)
    st = library().msda_backward_fused_workspace_size(ctypes.byref(dims), _value_dtype(value),
                                                      ctypes.byref(n))
    if st != 0:
        raise MsdaError(st, "msda_backward_fused_workspace_size")
    return n.value


def msda_backward_fused(value, spatial_shapes, level_start_index, reference_points,
                        sampling_offsets, attention_logits, grad_output, grad_value=None,
                        grad_reference_points=None, grad_sampling_offsets=None,
                        grad_attention_logits=None, needs=(True, True, True, True),
                        workspace=None, stream=None):
    """Fused backward (include/msda.h msda_backward_fused). Returns
    (grad_value, grad_reference_points, grad_sampling_offsets,
    grad_attention_logits), fp32, None where ``needs`` is False; given output
    tensors are written in place."""
    dev, dims = _common_fused(value, spatial_shapes, level_start_index, reference_points,
                              sampling_offsets, attention_logits)
    _check(grad_output, "grad_output", (torch.float32,), dev)
    if grad_output.numel() != dims.B * dims.Nq * dims.M * dims.D:
        raise ValueError("grad_output has the wrong number of elements")
    outs = []
    for need, given, shape, name in (
            (needs[0], grad_value, (dims.B, dims.Nv, dims.M, dims.D), "grad_value"),
            (needs[1], grad_reference_points, tuple(reference_points.shape),
             "grad_reference_points"),
            (needs[2], grad_sampling_offsets, tuple(sampling_offsets.shape),
             "grad_sampling_offsets"),
            (needs[3], grad_attention_logits, tuple(attention_logits.shape),
             "grad_attention_logits")):
        if not need:
            outs.append(None)
        elif given is None:
            outs.append(torch.empty(shape, dtype=torch.float32, device=dev))
        else:
            _check(given, name, (torch.float32,), dev)
            if tuple(given.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
            outs.append(given)
    n = msda_backward_fused_workspace_size(value, sampling_offsets)
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor on {dev}")
    st = library().msda_backward_fused(
        ctypes.byref(dims), _value_dtype(value), _ptr(value), _ptr(spatial_shapes),
        _ptr(level_start_index), _ptr(reference_points), _ptr(sampling_offsets),
        _ptr(attention_logits), _ptr(grad_output), *[_ptr(o) for o in outs], _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_backward_fused")
    return tuple(outs)


class MSDeformAttnFusedFunction(torch.autograd.Function):
    """Autograd wrapper of the fused front-end + core, both passes in HIP."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, reference_points,
                sampling_offsets, attention_logits):
        ctx.save_for_backward(value, spatial_shapes, level_start_index, reference_points,
                              sampling_offsets, attention_logits)
        return msda_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                                  sampling_offsets, attention_logits)

    @staticmethod
    def backward(ctx, grad_output):
        value, shapes, lsi, ref, off, logits = ctx.saved_tensors
        needs = (ctx.needs_input_grad[0], ctx.needs_input_grad[3], ctx.needs_input_grad[4],
                 ctx.needs_input_grad[5])
        gv, gr, go, gz = msda_backward_fused(value, shapes, lsi, ref, off, logits,
                                             grad_output.contiguous(), needs=needs)
        if gv is not None and value.dtype != torch.float32:
            gv = gv.to(value.dtype)
        return gv, None, None, gr, go, gz


def ms_deform_attn_fused(value, spatial_shapes, level_start_index, reference_points,
                         sampling_offsets, attention_logits):
    """Differentiable fused front-end + core: output [B, Nq, M*D]."""
    return MSDeformAttnFusedFunction.apply(value, spatial_shapes, level_start_index,
                                           reference_points, sampling_offsets, attention_logits)


# ----------------------------------------------------------------------------- linear layers
def _linear_sizes(x, weight):
    if weight.dim() != 2:
        raise ValueError("weight must be [out_features, in_features]")
    O, I = weight.shape
    if x.shape[-1] != I:
        raise ValueError("x's last dimension must equal in_features")
    return x.numel() // I if I else 0, I, O


def msda_linear_forward(x, weight, bias=None, output=None, stream=None):
    """y = x W^T + b on the matrix cores (include/msda.h msda_linear_forward).
    x [..., in], weight [out, in], bias [out] or None -> y [..., out], fp32."""
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    _check(x, "x", (torch.float32,), dev)
    _check(weight, "weight", (torch.float32,), dev)
    if bias is not None:
        _check(bias, "bias", (torch.float32,), dev)
    R, I, O = _linear_sizes(x, weight)
    if bias is not None and tuple(bias.shape) != (O,):
        raise ValueError("bias must be [out_features]")
    if output is None:
        output = torch.empty(tuple(x.shape[:-1]) + (O,), dtype=torch.float32, device=dev)
    else:
        _check(output, "output", (torch.float32,), dev)
        if output.numel() != R * O:
            raise ValueError("output has the wrong number of elements")
    st = library().msda_linear_forward(R, I, O, _ptr(x), _ptr(weight), _ptr(bias), _ptr(output),
                                       _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_linear_forward")
    return output


def msda_linear_backward_workspace_size(rows, in_features, out_features):
    n = ctypes.c_size_t(0)
    st = library().msda_linear_backward_workspace_size(rows, in_features, out_features,
                                                       ctypes.byref(n))
    if st != 0:
        raise MsdaError(st, "msda_linear_backward_workspace_size")
    return n.value


def msda_linear_backward(x, weight, grad_y, needs=(True, True, True), workspace=None,
                         stream=None):
    """Gradients of msda_linear_forward (include/msda.h msda_linear_backward):
    (grad_x, grad_weight, grad_bias), None where ``needs`` is False."""
    dev = x.device
    _check(x, "x", (torch.float32,), dev)
    _check(weight, "weight", (torch.float32,), dev)
    _check(grad_y, "grad_y", (torch.float32,), dev)
    R, I, O = _linear_sizes(x, weight)
    if grad_y.numel() != R * O:
        raise ValueError("grad_y has the wrong number of elements")
    gx = torch.empty_like(x) if needs[0] else None
    gw = torch.empty_like(weight) if needs[1] else None
    gb = torch.empty(O, dtype=torch.float32, device=dev) if needs[2] else None
    n = msda_linear_backward_workspace_size(R, I, O)
    if workspace is None and (needs[1] or needs[2]):
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().msda_linear_backward(R, I, O, _ptr(x), _ptr(weight), _ptr(grad_y), _ptr(gx),
                                        _ptr(gw), _ptr(gb), _ptr(workspace),
                                        ctypes.c_size_t(ws_bytes), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_linear_backward")
    return gx, gw, gb


# ----------------------------------------------------------------------------- the layer
def _layer_dims(query, input_flatten, spatial_shapes, n_heads, n_points):
    B, Nq, C = query.shape
    Bv, Nv, Cv = input_flatten.shape
    if (Bv, Cv) != (B, C):
        raise ValueError("query and input_flatten must share batch and channels")
    if C % n_heads:
        raise ValueError("channels must be a multiple of the head count")
    L = spatial_shapes.shape[0]
    return MsdaDims(B, Nv, n_heads, C // n_heads, L, Nq, n_points)


def _layer_params(params, dev):
    st = MsdaLayerParams()
    for n in LAYER_PARAMS:
        t = params.get(n)
        if t is not None:
            _check(t, n, (torch.float32,), dev)
        setattr(st, n, None if t is None else t.data_ptr())
    return st


def msda_layer_sizes(query, input_flatten, spatial_shapes, n_heads, n_points):
    """(saved bytes, workspace bytes) of the layer entry points."""
    dims = _layer_dims(query, input_flatten, spatial_shapes, n_heads, n_points)
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    for name, out in (("msda_layer_saved_size", a), ("msda_layer_workspace_size", b)):
        st = getattr(library(), name)(ctypes.byref(dims), ctypes.byref(out))
        if st != 0:
            raise MsdaError(st, name)
    return a.value, b.value


def msda_layer_forward(query, input_flatten, reference_points, spatial_shapes,
                       level_start_index, params, n_heads, n_points, output=None, saved=None,
                       stream=None):
    """MSDeformAttn layer forward (include/msda.h msda_layer_forward).
    params: dict of the eight tensors named in LAYER_PARAMS (biases may be
    None). Returns (output [B, Nq, C], saved), saved being the uint8 buffer
    the backward needs."""
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("query must be a GPU tensor")
    for t, n in ((query, "query"), (input_flatten, "input_flatten"),
                 (reference_points, "reference_points")):
        _check(t, n, (torch.float32,), dev)
    _check(spatial_shapes, "spatial_shapes", (torch.int64,), dev)
    _check(level_start_index, "level_start_index", (torch.int64,), dev)
    dims = _layer_dims(query, input_flatten, spatial_shapes, n_heads, n_points)
    if tuple(reference_points.shape) != (dims.B, dims.Nq, dims.L, 2):
        raise ValueError("reference_points must be [B, Nq, L, 2]")
    nsaved, _ = msda_layer_sizes(query, input_flatten, spatial_shapes, n_heads, n_points)
    if saved is None:
        saved = torch.empty(max(nsaved, 1), dtype=torch.uint8, device=dev)
    if output is None:
        output = torch.empty_like(query)
    pst = _layer_params(params, dev)
    st = library().msda_layer_forward(ctypes.byref(dims), _ptr(query), _ptr(input_flatten),
                                      _ptr(reference_points), _ptr(spatial_shapes),
                                      _ptr(level_start_index), ctypes.byref(pst), _ptr(output),
                                      _ptr(saved), ctypes.c_size_t(saved.numel()),
                                      _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_layer_forward")
    return output, saved


def msda_layer_backward(query, input_flatten, reference_points, spatial_shapes,
                        level_start_index, params, n_heads, n_points, saved, grad_output,
                        needs_inputs=(True, True, True), needs_params=True, grads=None,
                        workspace=None, stream=None):
    """Gradients of the layer (include/msda.h msda_layer_backward). Returns a
    dict: query, input_flatten, reference_points and the parameter names of
    LAYER_PARAMS (parameters that are None, or not needed, are absent).
    ``grads`` may hold preallocated output tensors under those names."""
    dev = query.device
    _check(grad_output, "grad_output", (torch.float32,), dev)
    dims = _layer_dims(query, input_flatten, spatial_shapes, n_heads, n_points)
    _, nws = msda_layer_sizes(query, input_flatten, spatial_shapes, n_heads, n_points)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    out = dict(grads or {})
    for need, name, like in zip(needs_inputs, ("query", "input_flatten", "reference_points"),
                                (query, input_flatten, reference_points)):
        if need and name not in out:
            out[name] = torch.empty_like(like)
        elif not need:
            out.pop(name, None)
    gst = MsdaLayerGrads()
    for n in LAYER_PARAMS:
        if needs_params and params.get(n) is not None:
            if n not in out:
                out[n] = torch.empty_like(params[n])
            setattr(gst, n, out[n].data_ptr())
        else:
            out.pop(n, None)
            setattr(gst, n, None)
    pst = _layer_params(params, dev)
    st = library().msda_layer_backward(
        ctypes.byref(dims), _ptr(query), _ptr(input_flatten), _ptr(reference_points),
        _ptr(spatial_shapes), _ptr(level_start_index), ctypes.byref(pst), _ptr(saved),
        ctypes.c_size_t(saved.numel()), _ptr(grad_output), _ptr(out.get("query")),
        _ptr(out.get("input_flatten")), _ptr(out.get("reference_points")), ctypes.byref(gst),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_layer_backward")
    return out


# ----------------------------------------------------------------------------- DCNv3
def dcn_output_size(H, W, kernel, stride=(1, 1), pad=(0, 0), dilation=(1, 1)):
    """Output rows and columns of the convolution grid."""
    return ((H + 2 * pad[0] - dilation[0] * (kernel[0] - 1) - 1) // stride[0] + 1,
            (W + 2 * pad[1] - dilation[1] * (kernel[1] - 1) - 1) // stride[1] + 1)


def _dcn_dims(inp, offset, kernel, stride, pad, dilation):
    if inp.dim() != 5:
        raise ValueError("input must be [B, H, W, G, D]")
    B, H, W, G, D = inp.shape
    if offset.dim() != 6 or offset.shape[-1] != 2 or offset.shape[0] != B or \
            offset.shape[3] != G or offset.shape[4] != kernel[0] * kernel[1]:
        raise ValueError("offset must be [B, H_out, W_out, G, kernel_h * kernel_w, 2]")
    Ho, Wo = offset.shape[1], offset.shape[2]
    return MsdaDcnDims(B, H, W, G, D, kernel[0], kernel[1], stride[0], stride[1], pad[0], pad[1],
                       dilation[0], dilation[1], Ho, Wo)


def _dcn_checks(inp, offset, mask, dev):
    _check(inp, "input", VALUE_DTYPES, dev)
    _check(offset, "offset", (torch.float32,), dev)
    _check(mask, "mask", (torch.float32,), dev)
    if tuple(mask.shape) != tuple(offset.shape[:5]):
        raise ValueError("mask must be [B, H_out, W_out, G, K]")


def msda_dcn_forward(inp, offset, mask, kernel, stride=(1, 1), pad=(0, 0), dilation=(1, 1),
                     output=None, stream=None):
    """Grouped single-level deformable aggregation (include/msda.h
    msda_dcn_forward): input [B,H,W,G,D], offset [B,Ho,Wo,G,K,2] (pixels),
    mask [B,Ho,Wo,G,K] -> output [B,Ho,Wo,G*D] (fp32)."""
    dev = inp.device
    if dev.type != "cuda":
        raise ValueError("input must be a GPU tensor")
    _dcn_checks(inp, offset, mask, dev)
    dims = _dcn_dims(inp, offset, kernel, stride, pad, dilation)
    if output is None:
        output = torch.empty((dims.B, dims.H_out, dims.W_out, dims.G * dims.D),
                             dtype=torch.float32, device=dev)
    st = library().msda_dcn_forward(ctypes.byref(dims), _value_dtype(inp), _ptr(inp),
                                    _ptr(offset), _ptr(mask), _ptr(output), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_dcn_forward")
    return output


def msda_dcn_backward_workspace_size(inp, offset, kernel, stride=(1, 1), pad=(0, 0),
                                     dilation=(1, 1)):
    dims = _dcn_dims(inp, offset, kernel, stride, pad, dilation)
    n = ctypes.c_size_t(0)
    st = library().msda_dcn_backward_workspace_size(ctypes.byref(dims), _value_dtype(inp),
                                                    ctypes.byref(n))
    if st != 0:
        raise MsdaError(st, "msda_dcn_backward_workspace_size")
    return n.value


def msda_dcn_backward(inp, offset, mask, grad_output, kernel, stride=(1, 1), pad=(0, 0),
                      dilation=(1, 1), needs=(True, True, True), grad_input=None,
                      grad_offset=None, grad_mask=None, workspace=None, stream=None):
    """Gradients of msda_dcn_forward: (grad_input [B,H,W,G,D] fp32,
    grad_offset, grad_mask), None where ``needs`` is False."""
    dev = inp.device
    _dcn_checks(inp, offset, mask, dev)
    _check(grad_output, "grad_output", (torch.float32,), dev)
    dims = _dcn_dims(inp, offset, kernel, stride, pad, dilation)
    if grad_output.numel() != dims.B * dims.H_out * dims.W_out * dims.G * dims.D:
        raise ValueError("grad_output has the wrong number of elements")
    outs = []
    for need, given, like in ((needs[0], grad_input, inp), (needs[1], grad_offset, offset),
                              (needs[2], grad_mask, mask)):
        if not need:
            outs.append(None)
        elif given is None:
            outs.append(torch.empty(like.shape, dtype=torch.float32, device=dev))
        else:
            outs.append(given)
    ws_bytes = 0
    if outs[0] is not None:
        n = msda_dcn_backward_workspace_size(inp, offset, kernel, stride, pad, dilation)
        if workspace is None:
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = library().msda_dcn_backward(ctypes.byref(dims), _value_dtype(inp), _ptr(inp),
                                     _ptr(offset), _ptr(mask), _ptr(grad_output),
                                     *[_ptr(o) for o in outs], _ptr(workspace),
                                     ctypes.c_size_t(ws_bytes), _stream(dev, stream))
    if st != 0:
        raise MsdaError(st, "msda_dcn_backward")
    return tuple(outs)
