"""Oracle for the MSDA forward core (test infrastructure only).

A plain, slow, single-threaded CPU implementation of the multi-scale
deformable attention core, written in C (``msda_oracle.c``) from the method's
definition and loaded here with ctypes.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import this package; the HIP library
never calls it and the two share no code.

``build()`` compiles ``liboracle.so`` with gcc.  ``msda_oracle_forward`` and
``msda3d_oracle_forward`` take the same tensors as the GPU entry points (on
the CPU), widen value and attention weights exactly to float64, keep the
sampling locations in float32 (the precision of the corner-index decision),
and return the float64 result ``[N, Lq, M*D]``.  ``msda_oracle_backward`` and
``msda3d_oracle_backward`` return the float64 gradients with respect to value,
sampling locations and attention weights for a given ``grad_out``.
``msda_oracle_forward_fused`` and ``msda3d_oracle_forward_fused`` add the
module's front end: softmax of attention logits (fp64) and location =
reference point + offset (fp32), then the same forward.
``msda_oracle_forward_pruned`` / ``msda3d_oracle_forward_pruned`` drop the
samples whose attention weight is below a threshold.  ``linear_oracle`` is the
fp64 projection y = x W^T + b.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msda_oracle.c")
# MSDA_ORACLE_SANITIZE=1 selects a build of the same source with
# AddressSanitizer and UndefinedBehaviorSanitizer (every finding aborts); the
# process must then preload the ASan runtime, e.g.
#   LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#   MSDA_ORACLE_SANITIZE=1 python -m pytest tests -m "not gpu"
SANITIZE = os.environ.get("MSDA_ORACLE_SANITIZE", "0") not in ("", "0")
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all"]
_lib = None


def build() -> str:
    """Compile the oracle into ``oracle/liboracle.so`` (always rebuilds; with
    MSDA_ORACLE_SANITIZE=1 the sanitizer build ``oracle/liboracle_san.so``)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", *(_SAN_FLAGS if SANITIZE else []), "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    ptr = ctypes.c_void_p
    for name in ("msda_oracle_forward", "msda3d_oracle_forward"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ptr] * 6 + [i64] * 7
    for name in ("msda_oracle_backward", "msda3d_oracle_backward"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ptr] * 9 + [i64] * 7
    for name in ("msda_oracle_forward_pruned", "msda3d_oracle_forward_pruned"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ptr] * 5 + [ctypes.c_double, ptr] + [i64] * 7
    for name in ("msda_oracle_forward_fused", "msda3d_oracle_forward_fused"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ptr] * 7 + [i64] * 7
    _lib = lib
    return lib


def _as_numpy(x, dtype):
    """Exact conversion of a torch tensor or array to a contiguous numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if np.dtype(dtype) == np.float64:
                x = x.to(torch.float64)  # exact for float32 and bfloat16
            x = x.contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    arr = np.ascontiguousarray(x)
    if arr.dtype != np.dtype(dtype):
        if np.dtype(dtype) == np.float32 and arr.dtype != np.float32:
            raise TypeError("sampling_locations must be float32")
        arr = np.ascontiguousarray(arr.astype(dtype))
    return arr


def _run(dims, value, spatial_shapes, level_start_index, sampling_locations,
         attention_weights, threshold=None):
    lib = _load()
    v = _as_numpy(value, np.float64)
    shapes = _as_numpy(spatial_shapes, np.int64)
    lsi = _as_numpy(level_start_index, np.int64)
    loc = _as_numpy(sampling_locations, np.float32)
    aw = _as_numpy(attention_weights, np.float64)
    if v.ndim != 4:
        raise ValueError("value must be [N, S, M, D]")
    N, S, M, D = v.shape
    if loc.ndim != 6 or loc.shape[-1] != dims:
        raise ValueError(f"sampling_locations must be [N, Lq, M, L, P, {dims}]")
    _, Lq, _, L, P, _ = loc.shape
    if aw.shape != loc.shape[:-1] or shapes.shape != (L, dims) or lsi.shape != (L,):
        raise ValueError("inconsistent shapes")
    out = np.empty((N, Lq, M * D), dtype=np.float64)
    if threshold is None:
        fn = lib.msda_oracle_forward if dims == 2 else lib.msda3d_oracle_forward
        rc = fn(v.ctypes.data, shapes.ctypes.data, lsi.ctypes.data, loc.ctypes.data,
                aw.ctypes.data, out.ctypes.data, N, S, M, D, Lq, L, P)
    else:
        fn = lib.msda_oracle_forward_pruned if dims == 2 else lib.msda3d_oracle_forward_pruned
        thr = float(np.float32(threshold))   # the threshold is an fp32 value
        rc = fn(v.ctypes.data, shapes.ctypes.data, lsi.ctypes.data, loc.ctypes.data,
                aw.ctypes.data, thr, out.ctypes.data, N, S, M, D, Lq, L, P)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out


def _run_backward(dims, value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out):
    lib = _load()
    v = _as_numpy(value, np.float64)
    shapes = _as_numpy(spatial_shapes, np.int64)
    lsi = _as_numpy(level_start_index, np.int64)
    loc = _as_numpy(sampling_locations, np.float32)
    aw = _as_numpy(attention_weights, np.float64)
    g = _as_numpy(grad_out, np.float64)
    N, S, M, D = v.shape
    _, Lq, _, L, P, _ = loc.shape
    if g.shape != (N, Lq, M * D):
        raise ValueError("grad_out must be [N, Lq, M*D]")
    gv = np.empty_like(v)
    gl = np.empty(loc.shape, dtype=np.float64)
    ga = np.empty(aw.shape, dtype=np.float64)
    fn = lib.msda_oracle_backward if dims == 2 else lib.msda3d_oracle_backward
    rc = fn(v.ctypes.data, shapes.ctypes.data, lsi.ctypes.data, loc.ctypes.data,
            aw.ctypes.data, g.ctypes.data, gv.ctypes.data, gl.ctypes.data, ga.ctypes.data,
            N, S, M, D, Lq, L, P)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return gv, gl, ga


def msda_oracle_backward(value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_out):
    """2D backward: returns (grad_value, grad_sampling_locations,
    grad_attention_weights), float64, shaped like value / locations / weights."""
    return _run_backward(2, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_out)


def msda3d_oracle_backward(value, spatial_shapes, level_start_index, sampling_locations,
                           attention_weights, grad_out):
    """3D backward (trilinear); see msda_oracle_backward."""
    return _run_backward(3, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_out)


def msda_oracle_forward_pruned(value, spatial_shapes, level_start_index, sampling_locations,
                               attention_weights, threshold) -> np.ndarray:
    """2D forward dropping samples whose attention weight is below ``threshold``
    (rounded to fp32); the kept weights are used as given."""
    return _run(2, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights, threshold)


def msda3d_oracle_forward_pruned(value, spatial_shapes, level_start_index, sampling_locations,
                                 attention_weights, threshold) -> np.ndarray:
    """3D counterpart of ``msda_oracle_forward_pruned``."""
    return _run(3, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights, threshold)


def msda_oracle_forward(value, spatial_shapes, level_start_index,
                        sampling_locations, attention_weights) -> np.ndarray:
    """2D oracle: value [N,S,M,D], shapes [L,2]=(H,W), locations [N,Lq,M,L,P,2]."""
    return _run(2, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights)


def msda3d_oracle_forward(value, spatial_shapes, level_start_index,
                          sampling_locations, attention_weights) -> np.ndarray:
    """3D oracle: value [N,S,M,D], shapes [L,3]=(Z,H,W), locations [...,3]."""
    return _run(3, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights)


def _run_fused(dims, value, spatial_shapes, level_start_index, reference_points,
               sampling_offsets, attention_logits):
    lib = _load()
    v = _as_numpy(value, np.float64)
    shapes = _as_numpy(spatial_shapes, np.int64)
    lsi = _as_numpy(level_start_index, np.int64)
    ref = _as_numpy(reference_points, np.float32)
    off = _as_numpy(sampling_offsets, np.float32)
    z = _as_numpy(attention_logits, np.float64)
    N, S, M, D = v.shape
    if off.ndim != 6 or off.shape[-1] != dims:
        raise ValueError(f"sampling_offsets must be [N, Lq, M, L, P, {dims}]")
    _, Lq, _, L, P, _ = off.shape
    if ref.shape != (N, Lq, dims) or z.shape != off.shape[:-1]:
        raise ValueError("inconsistent shapes")
    out = np.empty((N, Lq, M * D), dtype=np.float64)
    fn = lib.msda_oracle_forward_fused if dims == 2 else lib.msda3d_oracle_forward_fused
    rc = fn(v.ctypes.data, shapes.ctypes.data, lsi.ctypes.data, ref.ctypes.data,
            off.ctypes.data, z.ctypes.data, out.ctypes.data, N, S, M, D, Lq, L, P)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out


def msda_oracle_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                              sampling_offsets, attention_logits) -> np.ndarray:
    """2D forward with the front end: reference_points [N,Lq,2], offsets
    [N,Lq,M,L,P,2], logits [N,Lq,M,L,P]; returns float64 [N, Lq, M*D]."""
    return _run_fused(2, value, spatial_shapes, level_start_index, reference_points,
                      sampling_offsets, attention_logits)


def msda3d_oracle_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                                sampling_offsets, attention_logits) -> np.ndarray:
    """3D forward with the front end (reference points and offsets have 3
    components)."""
    return _run_fused(3, value, spatial_shapes, level_start_index, reference_points,
                      sampling_offsets, attention_logits)


def linear_oracle(x, weight, bias=None) -> np.ndarray:
    """Projection y = x @ weight^T + bias in float64 (inputs widened exactly):
    the per-pixel linear maps W'_m and W_m of the "Deformable Attention
    Module" equation and the query-side predictions of offsets and logits.
    A library matmul serves as the one step; no blocking or reordering."""
    xd = _as_numpy(x, np.float64)
    wd = _as_numpy(weight, np.float64)
    y = xd @ wd.T
    if bias is not None:
        y = y + _as_numpy(bias, np.float64)[None, :]
    return y
