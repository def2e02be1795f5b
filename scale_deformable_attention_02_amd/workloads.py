"""Seeded synthetic workloads for the MSDA core (forward and backward).

This module only draws inputs: it holds none of the sampling or interpolation
arithmetic, and both the GPU path's tests/benchmark and the oracle consume
exactly the tensors it returns.  No dataset or trained weights are involved;
the shapes and value distributions stand in for Deformable-DETR activations
(feature pyramid of a ~800x1333 image at strides 8..64) and for a 64^3 volume
pyramid.

Recipe (one ``torch.Generator`` on the CPU, seeded per workload, draws in this
order):
  1. value ~ N(0, 1) as float32 [N, S, M, D]; rounded to bfloat16 (RNE) when
     the workload's value dtype is bf16;
  2. reference points: for ``uniform`` workloads the sampling locations are
     drawn directly, U[lo, hi] per coordinate; for ``random_refs`` one
     reference point U[0, 1]^dims per (n, q); for ``pixel_centres`` query q is
     the q-th flattened pixel of the pyramid and its reference point is that
     pixel's centre ((j+0.5)/W, (i+0.5)/H[, (k+0.5)/Z]) in normalized units,
     reused at every level;
  3. offsets ~ N(0, sigma) per (n, q, m, l, p, coordinate) in normalized units,
     added to the reference point (float32);
  4. logits ~ N(0, 1) per (n, q, m, l, p); attention weights are their softmax
     over the L*P samples of each (n, q, m), taken in float64, stored float32.
``make_fused_inputs`` returns the draws of steps 2-4 before they are
combined (reference points, offsets, logits), for the forward with the fused
front end.  For a backward pass ``make_grad_out`` draws the output gradient
~ N(0, 1) from a generator of its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import torch

LEVELS_2D = ((100, 167), (50, 84), (25, 42), (13, 21))
LEVELS_3D = ((64, 64, 64), (32, 32, 32), (16, 16, 16), (8, 8, 8))


@dataclass(frozen=True)
class Workload:
    name: str
    dims: int                       # 2 (bilinear) or 3 (trilinear)
    N: int                          # batch
    shapes: Tuple[Tuple[int, ...], ...]  # per level (H, W) or (Z, H, W)
    Lq: Optional[int]               # queries per image; None means Lq = S
    M: int                          # heads
    D: int                          # channels per head
    P: int                          # points per level
    value_dtype: str = "f32"        # "f32" or "bf16"
    queries: str = "pixel_centres"  # "uniform", "random_refs", "pixel_centres"
    sigma: float = 0.02             # offset std (normalized units)
    box: Tuple[float, float] = (-0.1, 1.1)  # range of "uniform" locations
    seed: int = 1000
    description: str = field(default="", compare=False)
    out_dtype: str = "f32"          # "f32" or "bf16" (accumulation is fp32)

    @property
    def L(self) -> int:
        return len(self.shapes)

    @property
    def S(self) -> int:
        total = 0
        for shp in self.shapes:
            size = 1
            for e in shp:
                size *= e
            total += size
        return total

    @property
    def queries_per_image(self) -> int:
        return self.S if self.Lq is None else self.Lq

    @property
    def sampled_points(self) -> int:
        return self.N * self.queries_per_image * self.M * self.L * self.P

    @property
    def value_itemsize(self) -> int:
        return 2 if self.value_dtype == "bf16" else 4

    @property
    def out_itemsize(self) -> int:
        return 2 if self.out_dtype == "bf16" else 4

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", 2, 1, ((16, 16),), 64, 2, 8, 4, "f32", "uniform", 0.0,
        (-0.1, 1.1), 1001,
        "tiny single-scale fp32: 16x16 map, M=2, D=8, Lq=64, L=1, P=4, "
        "locations U[-0.1,1.1]^2"),
    "detr_encoder": Workload(
        "detr_encoder", 2, 2, LEVELS_2D, None, 8, 32, 4, "f32",
        "pixel_centres", 0.02, (0.0, 1.0), 1002,
        "Deformable-DETR encoder fp32: N=2, 4 levels, S=Lq=22223, M=8, D=32, "
        "L=4, P=4, pixel-centre refs + N(0,0.02)"),
    "detr_decoder": Workload(
        "detr_decoder", 2, 2, LEVELS_2D, 300, 8, 32, 4, "f32", "random_refs",
        0.05, (0.0, 1.0), 1003,
        "Deformable-DETR decoder fp32: N=2, S=22223, Lq=300, refs U[0,1]^2 + "
        "N(0,0.05)"),
    "detr_encoder_bf16_b8": Workload(
        "detr_encoder_bf16_b8", 2, 8, LEVELS_2D, None, 8, 32, 4, "bf16",
        "pixel_centres", 0.02, (0.0, 1.0), 1004,
        "Deformable-DETR encoder at scale, bf16 value, fp32 "
        "locations/weights/accumulation/out: N=8, S=Lq=22223"),
    "volume3d": Workload(
        "volume3d", 3, 1, LEVELS_3D, None, 8, 32, 4, "f32", "pixel_centres",
        0.02, (0.0, 1.0), 1005,
        "3D trilinear fp32: N=1, volumes 64^3..8^3, S=Lq=299520, M=8, D=32, "
        "L=4, P=4, voxel-centre refs + N(0,0.02)"),
}

# Order in which the configurations are listed (the tiny one first).
CONFIG_ORDER = ("tiny", "detr_encoder", "detr_decoder", "detr_encoder_bf16_b8",
                "volume3d")


def level_starts(shapes) -> list:
    """Offsets of each level in the flattened pyramid (prefix sums of sizes)."""
    starts, acc = [], 0
    for shp in shapes:
        starts.append(acc)
        size = 1
        for e in shp:
            size *= e
        acc += size
    return starts


def pixel_centre_refs(shapes, dims: int) -> torch.Tensor:
    """Normalized centre of every pixel of the pyramid, in flattened order.

    Returns float64 [S, dims] with component 0 = x (along W), 1 = y (along H),
    2 = z (along Z).
    """
    refs = []
    for shp in shapes:
        if dims == 2:
            H, W = shp
            i = torch.arange(H, dtype=torch.float64)
            j = torch.arange(W, dtype=torch.float64)
            ii, jj = torch.meshgrid(i, j, indexing="ij")
            r = torch.stack([(jj + 0.5) / W, (ii + 0.5) / H], dim=-1)
        else:
            Z, H, W = shp
            k = torch.arange(Z, dtype=torch.float64)
            i = torch.arange(H, dtype=torch.float64)
            j = torch.arange(W, dtype=torch.float64)
            kk, ii, jj = torch.meshgrid(k, i, j, indexing="ij")
            r = torch.stack([(jj + 0.5) / W, (ii + 0.5) / H, (kk + 0.5) / Z],
                            dim=-1)
        refs.append(r.reshape(-1, dims))
    return torch.cat(refs, dim=0)


def _draw(w: Workload, seed: Optional[int]):
    """The seeded draws of the recipe, in order: value, reference points (None
    for ``uniform`` workloads, whose locations are drawn directly), offsets or
    locations, logits."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    N, S, M, D, L, P, dims = w.N, w.S, w.M, w.D, w.L, w.P, w.dims
    Lq = w.queries_per_image

    value = torch.randn((N, S, M, D), generator=g, dtype=torch.float32)
    if w.value_dtype == "bf16":
        value = value.to(torch.bfloat16)
    elif w.value_dtype != "f32":
        raise ValueError(f"unknown value dtype {w.value_dtype!r}")

    loc_shape = (N, Lq, M, L, P, dims)
    ref = None
    if w.queries == "uniform":
        lo, hi = w.box
        off = torch.rand(loc_shape, generator=g, dtype=torch.float32) * (hi - lo) + lo
        if w.sigma:
            off = off + torch.randn(loc_shape, generator=g, dtype=torch.float32) * w.sigma
    else:
        if w.queries == "random_refs":
            ref = torch.rand((N, Lq, dims), generator=g, dtype=torch.float32)
        elif w.queries == "pixel_centres":
            if Lq != S:
                raise ValueError("pixel-centre queries need Lq == S")
            ref = pixel_centre_refs(w.shapes, dims).to(torch.float32)
            ref = ref.unsqueeze(0).expand(N, S, dims).contiguous()
        else:
            raise ValueError(f"unknown query layout {w.queries!r}")
        off = torch.randn(loc_shape, generator=g, dtype=torch.float32) * w.sigma

    logits = torch.randn((N, Lq, M, L * P), generator=g, dtype=torch.float32)
    shapes = torch.tensor(w.shapes, dtype=torch.int64).reshape(L, dims)
    starts = torch.tensor(level_starts(w.shapes), dtype=torch.int64)
    return value.contiguous(), shapes, starts, ref, off.contiguous(), logits


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw one batch of inputs for workload ``w`` on the CPU.

    Returns a dict with ``value`` ([N,S,M,D], float32 or bfloat16),
    ``spatial_shapes`` (int64 [L, dims]), ``level_start_index`` (int64 [L]),
    ``sampling_locations`` (float32 [N,Lq,M,L,P,dims]) and
    ``attention_weights`` (float32 [N,Lq,M,L,P]).
    """
    value, shapes, starts, ref, off, logits = _draw(w, seed)
    N, Lq, M, L, P, dims = off.shape
    if ref is None:
        loc = off
    else:
        loc = (ref.reshape(N, Lq, 1, 1, 1, dims) + off).contiguous()
    attw = torch.softmax(logits.to(torch.float64), dim=-1).to(torch.float32)
    attw = attw.reshape(N, Lq, M, L, P).contiguous()
    return {
        "value": value,
        "spatial_shapes": shapes,
        "level_start_index": starts,
        "sampling_locations": loc,
        "attention_weights": attw,
    }


def make_fused_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """The same draws as ``make_inputs`` before the front end: ``reference_points``
    (float32 [N,Lq,dims]; zeros for ``uniform`` workloads, whose offsets are
    then the drawn locations), ``sampling_offsets`` (float32 [N,Lq,M,L,P,dims])
    and ``attention_logits`` (float32 [N,Lq,M,L,P]), plus value, shapes and
    level starts.  reference + offset in fp32 equals make_inputs' locations
    bit for bit."""
    value, shapes, starts, ref, off, logits = _draw(w, seed)
    N, Lq, M, L, P, dims = off.shape
    if ref is None:
        ref = torch.zeros((N, Lq, dims), dtype=torch.float32)
    return {
        "value": value,
        "spatial_shapes": shapes,
        "level_start_index": starts,
        "reference_points": ref.contiguous(),
        "sampling_offsets": off,
        "attention_logits": logits.reshape(N, Lq, M, L, P).contiguous(),
    }


def make_grad_out(w: Workload, dtype: Optional[str] = None,
                  seed: Optional[int] = None) -> torch.Tensor:
    """Draw the output gradient for a backward pass of workload ``w``.

    ``grad_out`` ~ N(0, 1) as float32 [N, Lq, M*D] from its own generator
    (seed: the workload's + 7919 unless given), rounded to bfloat16 (RNE) when
    ``dtype`` is "bf16" (default: the workload's value dtype).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 7919 if seed is None else seed)
    grad = torch.randn((w.N, w.queries_per_image, w.M * w.D), generator=g,
                       dtype=torch.float32)
    dt = w.value_dtype if dtype is None else dtype
    if dt == "bf16":
        grad = grad.to(torch.bfloat16)
    elif dt != "f32":
        raise ValueError(f"unknown grad dtype {dt!r}")
    return grad.contiguous()


def make_linear_inputs(R: int, K: int, N: int, dtype: str = "bf16", seed: int = 2024,
                       bias: bool = True) -> Dict[str, torch.Tensor]:
    """Seeded operands of a projection y = x W^T + b: x ~ N(0, 1) [R, K],
    W ~ N(0, 1/K) [N, K] (unit-variance outputs), both rounded to bf16 (RNE)
    when ``dtype`` is "bf16"; b ~ N(0, 0.02) float32 [N] or None."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((R, K), generator=g, dtype=torch.float32)
    w = torch.randn((N, K), generator=g, dtype=torch.float32) / (K ** 0.5)
    b = torch.randn((N,), generator=g, dtype=torch.float32) * 0.02 if bias else None
    if dtype == "bf16":
        x, w = x.to(torch.bfloat16), w.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return {"x": x.contiguous(), "weight": w.contiguous(), "bias": b}
