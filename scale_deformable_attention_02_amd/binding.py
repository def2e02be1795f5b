"""Python binding of the C ABI in ``include/msda.h`` (argument marshalling only).

``msda_forward`` / ``msda3d_forward``, ``msda_forward_pruned`` /
``msda3d_forward_pruned``, ``msda_forward_fused`` / ``msda3d_forward_fused``
and ``msda_backward`` / ``msda3d_backward``, the projection ``msda_linear`` and
the visit-order builder ``msda_query_order``
take torch tensors that already live on the GPU, check
dtypes/shapes/contiguity, allocate outputs with torch when the caller passes
none, and call the same-named C entry point of ``libmsda.so`` on torch's
current HIP stream.  Every step of the computation
runs in the library's kernels.  If ``libmsda.so`` has not been built, the
first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsda.so")

MSDA_F32 = 0
MSDA_BF16 = 1

STATUS = {
    0: "MSDA_OK",
    1: "MSDA_ERR_NULL",
    2: "MSDA_ERR_DIM",
    3: "MSDA_ERR_DTYPE",
    4: "MSDA_ERR_UNSUPPORTED",
    5: "MSDA_ERR_ALIGN",
    6: "MSDA_ERR_OVERFLOW",
    7: "MSDA_ERR_LAUNCH",
}

# Every symbol include/msda.h and include/msda_calib.h declare.
EXPORTED = ("msda_forward", "msda3d_forward", "msda_forward_pruned", "msda3d_forward_pruned",
            "msda_forward_fused", "msda3d_forward_fused", "msda_backward", "msda3d_backward",
            "msda_linear", "msda_query_order", "msda_query_order_points", "msda_status_string",
            "msda_calib_gather_global", "msda_calib_gather_global_lds", "msda_calib_gather_lds",
            "msda_calib_stream")

_lib = None


class MsdaError(RuntimeError):
    """A non-zero msda_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load ``libmsda.so`` (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "scale_deformable_attention_02_amd._build.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    for name in ("msda_forward", "msda3d_forward"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int,
                       i64, i64, i64, i64, i64, i64, i64, vp, vp]
    for name in ("msda_forward_pruned", "msda3d_forward_pruned"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int,
                       i64, i64, i64, i64, i64, i64, i64, vp, vp]
    for name in ("msda_forward_fused", "msda3d_forward_fused"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                       i64, i64, i64, i64, i64, i64, i64, vp, vp]
    for name in ("msda_backward", "msda3d_backward"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                       i64, i64, i64, i64, i64, i64, i64, vp, vp]
    lib.msda_linear.restype = ctypes.c_int
    lib.msda_linear.argtypes = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
    lib.msda_query_order.restype = ctypes.c_int
    lib.msda_query_order.argtypes = [vp, i64, i64, ctypes.c_int, vp, i64, vp]
    lib.msda_query_order_points.restype = ctypes.c_int
    lib.msda_query_order_points.argtypes = [vp, i64, i64, vp, vp]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_status_string.argtypes = [ctypes.c_int]
    u64 = ctypes.c_uint64
    ci = ctypes.c_int
    lib.msda_calib_gather_global.restype = ci
    lib.msda_calib_gather_global.argtypes = [vp, u64, ci, ci, ci, vp, vp]
    lib.msda_calib_gather_global_lds.restype = ci
    lib.msda_calib_gather_global_lds.argtypes = [vp, u64, ci, ci, vp, vp]
    lib.msda_calib_gather_lds.restype = ci
    lib.msda_calib_gather_lds.argtypes = [vp, ci, ci, ci, vp, vp]
    lib.msda_calib_stream.restype = ci
    lib.msda_calib_stream.argtypes = [vp, u64, ci, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().msda_status_string(int(status)).decode()


def raw_call(dims: int, value_ptr: int, value_dtype: int, shapes_ptr: int,
             starts_ptr: int, loc_ptr: int, attw_ptr: int, out_ptr: int,
             out_dtype: int, N: int, S: int, M: int, D: int, Lq: int, L: int, P: int,
             stream: int = 0, order_ptr: int = 0) -> int:
    """Call the C entry point with raw pointers (``order_ptr``: the query
    order, 0 for none); returns the msda_status."""
    lib = load_library()
    fn = lib.msda_forward if dims == 2 else lib.msda3d_forward
    return fn(value_ptr, value_dtype, shapes_ptr, starts_ptr, loc_ptr, attw_ptr,
              out_ptr, out_dtype, N, S, M, D, Lq, L, P, order_ptr, stream)


def raw_pruned_call(dims: int, value_ptr: int, value_dtype: int, shapes_ptr: int,
                    starts_ptr: int, loc_ptr: int, attw_ptr: int, threshold: float, out_ptr: int,
                    out_dtype: int, N: int, S: int, M: int, D: int, Lq: int, L: int, P: int,
                    stream: int = 0, order_ptr: int = 0) -> int:
    """Call the pruned forward with raw pointers; returns the msda_status."""
    lib = load_library()
    fn = lib.msda_forward_pruned if dims == 2 else lib.msda3d_forward_pruned
    return fn(value_ptr, value_dtype, shapes_ptr, starts_ptr, loc_ptr, attw_ptr, threshold,
              out_ptr, out_dtype, N, S, M, D, Lq, L, P, order_ptr, stream)


def raw_fused_call(dims: int, value_ptr: int, value_dtype: int, shapes_ptr: int,
                   starts_ptr: int, ref_ptr: int, off_ptr: int, logits_ptr: int, out_ptr: int,
                   out_dtype: int, N: int, S: int, M: int, D: int, Lq: int, L: int, P: int,
                   stream: int = 0, order_ptr: int = 0) -> int:
    """Call the fused-front-end forward with raw pointers; returns the msda_status."""
    lib = load_library()
    fn = lib.msda_forward_fused if dims == 2 else lib.msda3d_forward_fused
    return fn(value_ptr, value_dtype, shapes_ptr, starts_ptr, ref_ptr, off_ptr, logits_ptr,
              out_ptr, out_dtype, N, S, M, D, Lq, L, P, order_ptr, stream)


def raw_backward_call(dims: int, value_ptr: int, value_dtype: int, shapes_ptr: int,
                      starts_ptr: int, loc_ptr: int, attw_ptr: int, grad_out_ptr: int,
                      grad_out_dtype: int, grad_value_ptr: int, grad_loc_ptr: int,
                      grad_attw_ptr: int, N: int, S: int, M: int, D: int, Lq: int, L: int,
                      P: int, stream: int = 0, order_ptr: int = 0) -> int:
    """Call the backward C entry point with raw pointers; returns the msda_status."""
    lib = load_library()
    fn = lib.msda_backward if dims == 2 else lib.msda3d_backward
    return fn(value_ptr, value_dtype, shapes_ptr, starts_ptr, loc_ptr, attw_ptr,
              grad_out_ptr, grad_out_dtype, grad_value_ptr, grad_loc_ptr, grad_attw_ptr,
              N, S, M, D, Lq, L, P, order_ptr, stream)


def _dtype_code(dtype: torch.dtype, what: str) -> int:
    if dtype == torch.float32:
        return MSDA_F32
    if dtype == torch.bfloat16:
        return MSDA_BF16
    raise TypeError(f"{what} must be float32 or bfloat16, got {dtype}")


def _check_inputs(dims, value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights):
    """Validate the forward inputs; returns (value dtype code, N, S, M, D, Lq, L, P)."""
    tensors = dict(value=value, spatial_shapes=spatial_shapes,
                   level_start_index=level_start_index,
                   sampling_locations=sampling_locations,
                   attention_weights=attention_weights)
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    code = _dtype_code(value.dtype, "value")
    if spatial_shapes.dtype != torch.int64 or level_start_index.dtype != torch.int64:
        raise TypeError("spatial_shapes and level_start_index must be int64")
    if sampling_locations.dtype != torch.float32 or attention_weights.dtype != torch.float32:
        raise TypeError("sampling_locations and attention_weights must be float32")
    if value.dim() != 4:
        raise ValueError("value must be [N, S, M, D]")
    N, S, M, D = value.shape
    if sampling_locations.dim() != 6 or sampling_locations.shape[-1] != dims:
        raise ValueError(f"sampling_locations must be [N, Lq, M, L, P, {dims}]")
    n2, Lq, m2, L, P, _ = sampling_locations.shape
    if (n2, m2) != (N, M) or attention_weights.shape != sampling_locations.shape[:-1]:
        raise ValueError("sampling_locations / attention_weights do not match value")
    if spatial_shapes.shape != (L, dims) or level_start_index.shape != (L,):
        raise ValueError("spatial_shapes / level_start_index do not match L")
    return code, N, S, M, D, Lq, L, P


def _order_ptr(query_order: Optional[torch.Tensor], Lq: int, device) -> int:
    """Pointer of a validated query order (int32 [Lq] on ``device``), or 0."""
    if query_order is None:
        return 0
    if (not query_order.is_cuda or query_order.device != device
            or query_order.dtype != torch.int32 or tuple(query_order.shape) != (Lq,)
            or not query_order.is_contiguous()):
        raise ValueError(f"query_order must be a contiguous int32 [{Lq}] tensor on value's "
                         "device")
    return query_order.data_ptr()


def _forward(dims: int, value: torch.Tensor, spatial_shapes: torch.Tensor,
             level_start_index: torch.Tensor, sampling_locations: torch.Tensor,
             attention_weights: torch.Tensor, out: Optional[torch.Tensor],
             out_dtype: Optional[torch.dtype],
             stream: Optional[torch.cuda.Stream],
             threshold: Optional[float] = None,
             query_order: Optional[torch.Tensor] = None) -> torch.Tensor:
    code, N, S, M, D, Lq, L, P = _check_inputs(dims, value, spatial_shapes, level_start_index,
                                               sampling_locations, attention_weights)
    if out is None:
        dt = value.dtype if out_dtype is None else out_dtype
        out = torch.empty((N, Lq, M * D), dtype=dt, device=value.device)
    elif (out.shape != (N, Lq, M * D) or not out.is_contiguous()
          or out.device != value.device or (out_dtype is not None and out.dtype != out_dtype)):
        raise ValueError("out must be a contiguous [N, Lq, M*D] tensor on value's device")
    out_code = _dtype_code(out.dtype, "out")
    order = _order_ptr(query_order, Lq, value.device)
    s = stream if stream is not None else torch.cuda.current_stream(value.device)
    if threshold is None:
        status = raw_call(dims, value.data_ptr(), code, spatial_shapes.data_ptr(),
                          level_start_index.data_ptr(), sampling_locations.data_ptr(),
                          attention_weights.data_ptr(), out.data_ptr(), out_code,
                          N, S, M, D, Lq, L, P, s.cuda_stream, order)
    else:
        status = raw_pruned_call(dims, value.data_ptr(), code, spatial_shapes.data_ptr(),
                                 level_start_index.data_ptr(), sampling_locations.data_ptr(),
                                 attention_weights.data_ptr(), float(threshold), out.data_ptr(),
                                 out_code, N, S, M, D, Lq, L, P, s.cuda_stream, order)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return out


def msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, out=None, out_dtype=None, stream=None,
                 query_order=None) -> torch.Tensor:
    """2D MSDA forward: value [N,S,M,D] (fp32/bf16), spatial_shapes [L,2]=(H,W),
    level_start_index [L], sampling_locations [N,Lq,M,L,P,2], attention_weights
    [N,Lq,M,L,P]; returns [N, Lq, M*D].  The output dtype is ``out``'s, else
    ``out_dtype``, else value's (fp32 accumulation either way; bf16 output is
    rounded to nearest-even).  ``query_order`` (int32 [Lq] on the GPU, a
    permutation, e.g. from ``msda_query_order``) sets the order in which the
    queries are visited; the result is the same.  Asynchronous on ``stream``
    (default: torch's current stream)."""
    return _forward(2, value, spatial_shapes, level_start_index, sampling_locations,
                    attention_weights, out, out_dtype, stream, query_order=query_order)


def msda3d_forward(value, spatial_shapes, level_start_index, sampling_locations,
                   attention_weights, out=None, out_dtype=None, stream=None,
                   query_order=None) -> torch.Tensor:
    """3D MSDA forward (trilinear): spatial_shapes [L,3]=(Z,H,W), locations
    [N,Lq,M,L,P,3] = (x, y, z); otherwise as ``msda_forward``."""
    return _forward(3, value, spatial_shapes, level_start_index, sampling_locations,
                    attention_weights, out, out_dtype, stream, query_order=query_order)


def _backward(dims, value, spatial_shapes, level_start_index, sampling_locations,
              attention_weights, grad_out, grad_value, grad_sampling_locations,
              grad_attention_weights, stream, query_order=None):
    code, N, S, M, D, Lq, L, P = _check_inputs(dims, value, spatial_shapes, level_start_index,
                                               sampling_locations, attention_weights)
    if not grad_out.is_cuda or not grad_out.is_contiguous() or grad_out.shape != (N, Lq, M * D):
        raise ValueError("grad_out must be a contiguous [N, Lq, M*D] GPU tensor")
    gcode = _dtype_code(grad_out.dtype, "grad_out")
    dev = value.device

    def _out(t, shape, name):
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=dev)
        if (t.dtype != torch.float32 or tuple(t.shape) != tuple(shape)
                or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous float32 {tuple(shape)} tensor")
        return t

    gv = _out(grad_value, (N, S, M, D), "grad_value")
    gl = _out(grad_sampling_locations, tuple(sampling_locations.shape),
              "grad_sampling_locations")
    ga = _out(grad_attention_weights, tuple(attention_weights.shape), "grad_attention_weights")
    order = _order_ptr(query_order, Lq, dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    status = raw_backward_call(dims, value.data_ptr(), code, spatial_shapes.data_ptr(),
                               level_start_index.data_ptr(), sampling_locations.data_ptr(),
                               attention_weights.data_ptr(), grad_out.data_ptr(), gcode,
                               gv.data_ptr(), gl.data_ptr(), ga.data_ptr(),
                               N, S, M, D, Lq, L, P, s.cuda_stream, order)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return gv, gl, ga


def msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out, grad_value=None,
                  grad_sampling_locations=None, grad_attention_weights=None,
                  stream=None, query_order=None):
    """2D MSDA backward: given ``grad_out`` [N, Lq, M*D] (fp32 or bf16) returns
    float32 ``(grad_value [N,S,M,D], grad_sampling_locations [N,Lq,M,L,P,2],
    grad_attention_weights [N,Lq,M,L,P])``; all three are overwritten (passed
    tensors are reused).  grad_value is accumulated with fp32 atomics, so its
    last bits may differ between runs.  ``query_order`` as in
    ``msda_forward``.  Asynchronous on ``stream``."""
    return _backward(2, value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, grad_out, grad_value, grad_sampling_locations,
                     grad_attention_weights, stream, query_order)


def msda3d_backward(value, spatial_shapes, level_start_index, sampling_locations,
                    attention_weights, grad_out, grad_value=None,
                    grad_sampling_locations=None, grad_attention_weights=None,
                    stream=None, query_order=None):
    """3D MSDA backward (trilinear); see ``msda_backward``."""
    return _backward(3, value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, grad_out, grad_value, grad_sampling_locations,
                     grad_attention_weights, stream, query_order)


def msda_forward_pruned(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights, threshold, out=None, out_dtype=None,
                        stream=None, query_order=None) -> torch.Tensor:
    """2D MSDA forward with probability-aware point pruning: samples whose
    attention weight is below ``threshold`` (an fp32 value) are skipped, the
    others keep their weights (no renormalisation); otherwise as
    ``msda_forward``."""
    return _forward(2, value, spatial_shapes, level_start_index, sampling_locations,
                    attention_weights, out, out_dtype, stream, threshold, query_order)


def msda3d_forward_pruned(value, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, threshold, out=None, out_dtype=None,
                          stream=None, query_order=None) -> torch.Tensor:
    """3D counterpart of ``msda_forward_pruned``."""
    return _forward(3, value, spatial_shapes, level_start_index, sampling_locations,
                    attention_weights, out, out_dtype, stream, threshold, query_order)


def _forward_fused(dims, value, spatial_shapes, level_start_index, reference_points,
                   sampling_offsets, attention_logits, out, out_dtype, stream,
                   query_order=None):
    code, N, S, M, D, Lq, L, P = _check_inputs(dims, value, spatial_shapes, level_start_index,
                                               sampling_offsets, attention_logits)
    if (not reference_points.is_cuda or not reference_points.is_contiguous()
            or reference_points.dtype != torch.float32
            or tuple(reference_points.shape) != (N, Lq, dims)):
        raise ValueError(f"reference_points must be a contiguous float32 [N, Lq, {dims}] "
                         "GPU tensor")
    if out is None:
        dt = value.dtype if out_dtype is None else out_dtype
        out = torch.empty((N, Lq, M * D), dtype=dt, device=value.device)
    elif (out.shape != (N, Lq, M * D) or not out.is_contiguous()
          or out.device != value.device or (out_dtype is not None and out.dtype != out_dtype)):
        raise ValueError("out must be a contiguous [N, Lq, M*D] tensor on value's device")
    out_code = _dtype_code(out.dtype, "out")
    order = _order_ptr(query_order, Lq, value.device)
    s = stream if stream is not None else torch.cuda.current_stream(value.device)
    status = raw_fused_call(dims, value.data_ptr(), code, spatial_shapes.data_ptr(),
                            level_start_index.data_ptr(), reference_points.data_ptr(),
                            sampling_offsets.data_ptr(), attention_logits.data_ptr(),
                            out.data_ptr(), out_code, N, S, M, D, Lq, L, P, s.cuda_stream,
                            order)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return out


def msda_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                       sampling_offsets, attention_logits, out=None, out_dtype=None,
                       stream=None, query_order=None) -> torch.Tensor:
    """2D MSDA forward with the front end fused: attention weights = softmax of
    ``attention_logits`` [N,Lq,M,L,P] over the L*P samples of each (n, q, m),
    locations = ``reference_points`` [N,Lq,2] + ``sampling_offsets``
    [N,Lq,M,L,P,2] (fp32); otherwise as ``msda_forward``."""
    return _forward_fused(2, value, spatial_shapes, level_start_index, reference_points,
                          sampling_offsets, attention_logits, out, out_dtype, stream,
                          query_order)


def msda3d_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                         sampling_offsets, attention_logits, out=None, out_dtype=None,
                         stream=None, query_order=None) -> torch.Tensor:
    """3D counterpart of ``msda_forward_fused`` (3-component points)."""
    return _forward_fused(3, value, spatial_shapes, level_start_index, reference_points,
                          sampling_offsets, attention_logits, out, out_dtype, stream,
                          query_order)


def raw_linear_call(x_ptr: int, x_dtype: int, w_ptr: int, bias_ptr: int, y_ptr: int,
                    y_dtype: int, R: int, K: int, N: int, stream: int = 0) -> int:
    """Call msda_linear with raw pointers; returns the msda_status."""
    return load_library().msda_linear(x_ptr, x_dtype, w_ptr, bias_ptr, y_ptr, y_dtype,
                                      R, K, N, stream)


def msda_linear(x, weight, bias=None, out=None, out_dtype=None, stream=None) -> torch.Tensor:
    """Projection ``out = x @ weight.T + bias`` on the matrix cores: x [R, K]
    and weight [N, K] both float32 or both bfloat16 (contiguous GPU tensors),
    bias float32 [N] or None; out [R, N] of ``out_dtype`` (default x's).
    K must be a multiple of 32."""
    for name, t in (("x", x), ("weight", weight)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D GPU tensor")
    if x.dtype != weight.dtype:
        raise TypeError("x and weight must have the same dtype")
    code = _dtype_code(x.dtype, "x")
    R, K = x.shape
    N, K2 = weight.shape
    if K2 != K:
        raise ValueError("weight must be [N, K] with x's K")
    if bias is not None and (not bias.is_cuda or bias.dtype != torch.float32
                             or tuple(bias.shape) != (N,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [N] GPU tensor")
    if out is None:
        out = torch.empty((R, N), dtype=x.dtype if out_dtype is None else out_dtype,
                          device=x.device)
    elif tuple(out.shape) != (R, N) or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous [R, N] tensor on x's device")
    ycode = _dtype_code(out.dtype, "out")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    status = raw_linear_call(x.data_ptr(), code, weight.data_ptr(),
                             0 if bias is None else bias.data_ptr(), out.data_ptr(), ycode,
                             R, K, N, s.cuda_stream)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return out


def raw_query_order_call(shapes_ptr: int, L: int, dims: int, level_major: int, order_ptr: int,
                         S: int, stream: int = 0) -> int:
    """Call msda_query_order with raw pointers (shapes on the host); returns
    the msda_status."""
    return load_library().msda_query_order(shapes_ptr, L, dims, level_major, order_ptr, S,
                                           stream)


def msda_query_order(spatial_shapes, level_major: bool = True, device=None, out=None,
                     stream=None) -> torch.Tensor:
    """Visit order for queries that are the pyramid's pixel centres (query s is
    pixel s): int32 [S] on ``device`` (default: the current GPU), the pixels
    ranked by the Z-order key of their normalized centre on a 2^10 grid per
    axis, level by level (``level_major``) or with the levels interleaved.
    ``spatial_shapes`` is [L, 2] = (H, W) or [L, 3] = (Z, H, W) (a tensor on
    any device, or nested sequences); it is read on the host."""
    shapes = torch.as_tensor(spatial_shapes, dtype=torch.int64).cpu().contiguous()
    if shapes.dim() != 2 or shapes.shape[1] not in (2, 3):
        raise ValueError("spatial_shapes must be [L, 2] or [L, 3]")
    L, dims = shapes.shape
    S = int(torch.prod(shapes, dim=1).sum())
    if out is None:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        out = torch.empty((S,), dtype=torch.int32, device=dev)
    elif (not out.is_cuda or out.dtype != torch.int32 or tuple(out.shape) != (S,)
          or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous int32 [{S}] GPU tensor")
    s = stream if stream is not None else torch.cuda.current_stream(out.device)
    status = raw_query_order_call(shapes.data_ptr(), L, dims, 1 if level_major else 0,
                                  out.data_ptr(), S, s.cuda_stream)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return out


def raw_query_order_points_call(points_ptr: int, Lq: int, dims: int, order_ptr: int,
                                stream: int = 0) -> int:
    """Call msda_query_order_points with raw device pointers; returns the
    msda_status."""
    return load_library().msda_query_order_points(points_ptr, Lq, dims, order_ptr, stream)


def msda_query_order_points(points, out=None, stream=None) -> torch.Tensor:
    """Visit order for queries given by one point each (data-dependent
    reference points): int32 [Lq], the queries ranked by (Z-order key of the
    point's cell on a 2^16 (2D) or 2^10 (3D) grid per axis, query index).
    ``points`` is a float32 GPU tensor [Lq, 2] = (x, y) or [Lq, 3] =
    (x, y, z) in normalized coordinates, at most 2^21 of them (the rank
    count is quadratic).  The order is one permutation for all images of a
    call, so pass the points of the image it should follow."""
    if (not isinstance(points, torch.Tensor) or not points.is_cuda or points.dim() != 2
            or points.shape[1] not in (2, 3) or points.dtype != torch.float32):
        raise ValueError("points must be a float32 GPU tensor [Lq, 2] or [Lq, 3]")
    points = points.contiguous()
    Lq, dims = points.shape
    if out is None:
        out = torch.empty((Lq,), dtype=torch.int32, device=points.device)
    elif (not out.is_cuda or out.dtype != torch.int32 or tuple(out.shape) != (Lq,)
          or not out.is_contiguous() or out.device != points.device):
        raise ValueError(f"out must be a contiguous int32 [{Lq}] tensor on the points' device")
    s = stream if stream is not None else torch.cuda.current_stream(points.device)
    status = raw_query_order_points_call(points.data_ptr(), Lq, dims, out.data_ptr(),
                                         s.cuda_stream)
    if status != 0:
        raise MsdaError(status, status_string(status))
    return out


# ---------------------------------------------------------------------------
# Gather-ceiling calibration (include/msda_calib.h): measurement kernels, not
# part of the operator.  Each call enqueues one launch on torch's current
# stream and returns the bytes it moves; the caller times it.
# ---------------------------------------------------------------------------
CALIB_THREADS = 256


def _calib_check(status: int, name: str):
    if status != 0:
        raise MsdaError(status, f"{name}: {status_string(status)}")


def calib_gather_global(buf: torch.Tensor, window_bytes: int, blocks: int, iters: int,
                        sink: torch.Tensor, lanes_per_row: int = 8) -> int:
    """Random 128-byte rows from the first ``window_bytes`` of ``buf``, read
    by 8 lanes with one load each or by 4 lanes with two loads each."""
    lib = load_library()
    assert buf.is_cuda and sink.is_cuda and buf.numel() * buf.element_size() >= window_bytes
    assert sink.numel() * sink.element_size() >= blocks * CALIB_THREADS * 16
    st = lib.msda_calib_gather_global(buf.data_ptr(), window_bytes, lanes_per_row, blocks, iters,
                                      sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _calib_check(st, "msda_calib_gather_global")
    return blocks * CALIB_THREADS * iters * 16


def calib_gather_global_lds(buf: torch.Tensor, window_bytes: int, blocks: int, iters: int,
                            sink: torch.Tensor) -> int:
    """The rows of ``calib_gather_global`` (8 lanes per row) delivered into
    LDS by the loads' LDS mode, then read back from LDS."""
    lib = load_library()
    assert buf.is_cuda and sink.is_cuda and buf.numel() * buf.element_size() >= window_bytes
    assert sink.numel() * sink.element_size() >= blocks * CALIB_THREADS * 16
    st = lib.msda_calib_gather_global_lds(buf.data_ptr(), window_bytes, blocks, iters,
                                          sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _calib_check(st, "msda_calib_gather_global_lds")
    return blocks * CALIB_THREADS * iters * 16


def calib_gather_lds(fill: torch.Tensor, mode: int, blocks: int, iters: int,
                     sink: torch.Tensor) -> int:
    """16-byte reads per lane from a 64 KB LDS array in the pattern ``mode``
    (0 random rows, 1 x-adjacent row pairs, 2 broadcast, 3 and 4 half rows on
    the same or opposite banks, 5 and 6 the corner rows of bilinear samples
    with and without swapped halves; include/msda_calib.h)."""
    lib = load_library()
    assert fill.is_cuda and sink.is_cuda and fill.numel() * fill.element_size() >= 65664
    assert sink.numel() * sink.element_size() >= blocks * CALIB_THREADS * 16
    st = lib.msda_calib_gather_lds(fill.data_ptr(), mode, blocks, iters, sink.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    _calib_check(st, "msda_calib_gather_lds")
    return blocks * CALIB_THREADS * iters * 16


def calib_stream(buf: torch.Tensor, nbytes: int, blocks: int, sink: torch.Tensor) -> int:
    """A coalesced read of ``nbytes`` of ``buf``."""
    lib = load_library()
    assert buf.is_cuda and sink.is_cuda and buf.numel() * buf.element_size() >= nbytes
    assert sink.numel() * sink.element_size() >= blocks * CALIB_THREADS * 16
    st = lib.msda_calib_stream(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    _calib_check(st, "msda_calib_stream")
    return nbytes
