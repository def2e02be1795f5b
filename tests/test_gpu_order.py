"""GPU: the visit order.

The order builder against the oracle's sort (integer work: bit-exact), and
every forward and backward entry point called with an order against the same
call without one.  The order changes only which wave visits a query, never the
arithmetic of a query, so every forward output and the location and weight
gradients must be bit-identical; grad_value (fp32 atomics) is checked against
the oracle with the backward's own bounds.  Orders come from the builder for
pixel-centre queries, and from the points builder (on the first image's first
sampling locations) or a random permutation otherwise; the cases cover
the direct and the LDS-staged forward kernels, the de-duplicating backward,
2D and 3D, fp32 and bf16.
"""
import numpy as np
import pytest
import torch

from oracle.order import points_order_oracle, query_order_oracle
from scale_deformable_attention_02_amd import (msda3d_backward, msda3d_forward,
                                               msda3d_forward_fused, msda3d_forward_pruned,
                                               msda_backward, msda_forward, msda_forward_fused,
                                               msda_forward_pruned, msda_query_order,
                                               msda_query_order_points)
from scale_deformable_attention_02_amd.workloads import (CONFIGS, Workload, make_fused_inputs,
                                                         make_grad_out, make_inputs)
from test_gpu_backward import check_backward
from test_gpu_parity import assert_parity, oracle_fwd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)


ORDER_SHAPES = [
    ((100, 150), (50, 75), (25, 38), (13, 19)),                 # DETR encoder pyramid
    ((64, 64, 64), (32, 32, 32), (16, 16, 16), (8, 8, 8)),      # 3D volume pyramid
    ((1, 1),),
    ((7, 1), (1, 9), (3, 3)),
    ((1, 1500), (2, 700)),            # wider than the 1024-cell grid
    ((1023, 3), (5, 1025)),
    ((5, 3, 7), (1, 1, 1), (2, 9, 4)),
    ((6, 10),) * 16,                  # 16 levels
]


@pytest.mark.parametrize("shapes", ORDER_SHAPES, ids=lambda s: f"L{len(s)}-{len(s[0])}d-{s[0]}")
@pytest.mark.parametrize("level_major", [True, False])
def test_order_builder_matches_oracle(shapes, level_major):
    _log(f"[order] builder {shapes} level_major={level_major}")
    got = msda_query_order(shapes, level_major, device=DEV)
    torch.cuda.synchronize()
    want = query_order_oracle(shapes, level_major)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), want)


def test_order_builder_reuses_out_and_runs_on_a_side_stream():
    shapes = ((20, 33), (10, 17))
    out = torch.full((20 * 33 + 10 * 17,), -1, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        got = msda_query_order(shapes, False, out=out, stream=side)
    side.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert np.array_equal(out.cpu().numpy(), query_order_oracle(shapes, False))


def _points(n, dims, seed):
    """Points of every kind the builder must rank like the oracle: uniform,
    clustered (equal cells), exact duplicates, values on cell edges, outside
    [0, 1], infinite and NaN."""
    g = np.random.default_rng(seed)
    pts = g.random((n, dims)).astype(np.float32)
    if n >= 64:
        pts[: n // 4] = (0.5 + 1e-4 * g.standard_normal((n // 4, dims))).astype(np.float32)
        pts[n // 4: n // 4 + 8] = pts[0]
        pts[40] = 0.25
        pts[41] = (-0.5, 1.5, 0.75)[:dims]
        pts[42] = (np.inf, -np.inf, np.nan)[:dims]
        pts[43] = (np.nan, 0.1, 2.0)[:dims]
        pts[44] = 1.0
    return pts


@pytest.mark.parametrize("dims", [2, 3])
@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 3001, 22223])
def test_points_order_builder_matches_oracle(dims, n):
    _log(f"[order] points builder dims={dims} n={n}")
    pts = _points(n, dims, 100 + n + dims)
    got = msda_query_order_points(torch.from_numpy(pts).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.int64), points_order_oracle(pts))


def test_points_order_builder_reuses_out_on_a_side_stream():
    pts = torch.from_numpy(_points(1000, 2, 5)).to(DEV)
    out = torch.full((1000,), -1, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        got = msda_query_order_points(pts, out=out, stream=side)
    side.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert np.array_equal(out.cpu().numpy(), points_order_oracle(pts.cpu().numpy()))


# Cases: (label, workload).  Pixel-centre workloads take the builder's orders,
# the others the points builder's order and a random permutation.
CASES = [
    ("2d-direct-pixel", Workload("o1", 2, 2, ((20, 33), (10, 17), (5, 9), (3, 5)), None, 8, 32,
                                 4, "f32", "pixel_centres", 0.03, (0, 1), 31)),
    ("2d-direct-refs", Workload("o2", 2, 2, ((20, 33), (10, 17), (5, 9), (3, 5)), 301, 8, 32,
                                4, "f32", "random_refs", 0.05, (0, 1), 32)),
    ("2d-staged-pixel", Workload("o3", 2, 2, ((60, 90), (30, 45), (15, 23), (8, 12)), None, 8,
                                 32, 4, "f32", "pixel_centres", 0.03, (0, 1), 33)),
    ("2d-staged-bf16", Workload("o4", 2, 2, ((60, 90), (30, 45), (15, 23), (8, 12)), None, 8,
                                32, 4, "bf16", "pixel_centres", 0.03, (0, 1), 34)),
    ("3d-pixel", Workload("o5", 3, 2, ((16, 16, 16), (8, 8, 8), (4, 4, 4)), None, 8, 32, 4,
                          "f32", "pixel_centres", 0.03, (0, 1), 35)),
    ("3d-refs-bf16", Workload("o6", 3, 1, ((6, 7, 9), (3, 4, 5)), 111, 8, 32, 3, "bf16",
                              "random_refs", 0.05, (0, 1), 36)),
]


def _orders(w):
    if w.queries == "pixel_centres":
        return [("morton-levels", msda_query_order(w.shapes, True, device=DEV)),
                ("morton-interleaved", msda_query_order(w.shapes, False, device=DEV))]
    g = torch.Generator().manual_seed(w.seed)
    perm = torch.randperm(w.queries_per_image, generator=g).to(torch.int32)
    # the first image's first sampling location of every query (head 0,
    # level 0, point 0) as its point
    loc = make_inputs(w)["sampling_locations"][0, :, 0, 0, 0, :].contiguous()
    return [("points", msda_query_order_points(loc.to(DEV))), ("random", perm.to(DEV))]


def _to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_forward_entry_points_with_an_order(label, w):
    dims = w.dims
    inp = make_inputs(w)
    d = _to_dev(inp)
    fwd = msda_forward if dims == 2 else msda3d_forward
    pruned = msda_forward_pruned if dims == 2 else msda3d_forward_pruned
    fused = msda_forward_fused if dims == 2 else msda3d_forward_fused
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
            d["attention_weights"])
    fin = _to_dev(make_fused_inputs(w))
    fargs = (fin["value"], fin["spatial_shapes"], fin["level_start_index"],
             fin["reference_points"], fin["sampling_offsets"], fin["attention_logits"])
    out_dtypes = [torch.float32] + ([torch.bfloat16] if w.value_dtype == "bf16" else [])
    ref = oracle_fwd(dims, inp)
    for name, order in _orders(w):
        _log(f"[order] forward {label} {name}")
        for odt in out_dtypes:
            base = fwd(*args, out_dtype=odt)
            got = fwd(*args, out_dtype=odt, query_order=order)
            torch.cuda.synchronize()
            assert torch.equal(got, base), (name, odt)
            assert_parity(got, ref)
            base = pruned(*args, 0.05, out_dtype=odt)
            got = pruned(*args, 0.05, out_dtype=odt, query_order=order)
            torch.cuda.synchronize()
            assert torch.equal(got, base), (name, odt, "pruned")
            base = fused(*fargs, out_dtype=odt)
            got = fused(*fargs, out_dtype=odt, query_order=order)
            torch.cuda.synchronize()
            assert torch.equal(got, base), (name, odt, "fused")


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_backward_with_an_order(label, w):
    dims = w.dims
    inp = make_inputs(w)
    grad = make_grad_out(w)
    d = _to_dev(inp)
    g = grad.to(DEV)
    bwd = msda_backward if dims == 2 else msda3d_backward
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
            d["attention_weights"], g)
    _, gl0, ga0 = bwd(*args)
    for name, order in _orders(w):
        _log(f"[order] backward {label} {name}")
        gv, gl, ga = bwd(*args, query_order=order)
        torch.cuda.synchronize()
        assert torch.equal(gl, gl0) and torch.equal(ga, ga0), name
        check_backward(dims, inp, grad, (gv, gl, ga))


def test_encoder_workload_with_orders_at_full_size():
    # the full DETR encoder workload: every forward output bitwise against the
    # unordered call, and sampled rows against the oracle
    w = CONFIGS["detr_encoder"]
    inp = make_inputs(w)
    d = _to_dev(inp)
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
            d["attention_weights"])
    base = msda_forward(*args)
    for level_major in (True, False):
        order = msda_query_order(w.shapes, level_major, device=DEV)
        got = msda_forward(*args, query_order=order)
        torch.cuda.synchronize()
        _log(f"[order] encoder level_major={level_major}")
        assert torch.equal(got, base)
    rows = torch.randperm(w.queries_per_image, generator=torch.Generator().manual_seed(5))[:64]
    sub = dict(inp, sampling_locations=inp["sampling_locations"][:, rows].contiguous(),
               attention_weights=inp["attention_weights"][:, rows].contiguous())
    assert_parity(got[:, rows.to(DEV)], oracle_fwd(2, sub))


@pytest.mark.parametrize("dims", [2, 3])
def test_entries_outside_the_queries_are_clamped(dims):
    # every entry past the end (or negative) reads as the last query: only its
    # output row is written, and nothing outside the tensors is touched
    shapes = ((9, 11), (5, 6)) if dims == 2 else ((5, 6, 7), (2, 3, 4))
    w = Workload("clamp", dims, 2, shapes, 37, 4, 16, 2, "f32", "random_refs", 0.05,
                 (0, 1), 41)
    inp = make_inputs(w)
    d = _to_dev(inp)
    fwd = msda_forward if dims == 2 else msda3d_forward
    bwd = msda_backward if dims == 2 else msda3d_backward
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
            d["attention_weights"])
    order = torch.full((37,), 2 ** 31 - 1, dtype=torch.int32)
    order[::2] = -5
    order = order.to(DEV)
    base = fwd(*args)
    out = torch.full_like(base, float("nan"))
    fwd(*args, out=out, query_order=order)
    torch.cuda.synchronize()
    assert torch.equal(out[:, -1], base[:, -1])
    assert torch.isnan(out[:, :-1]).all()
    g = make_grad_out(w).to(DEV)
    _, gl0, ga0 = bwd(*args, g)
    gl = torch.full_like(gl0, float("nan"))
    ga = torch.full_like(ga0, float("nan"))
    bwd(*args, g, grad_sampling_locations=gl, grad_attention_weights=ga, query_order=order)
    torch.cuda.synchronize()
    assert torch.equal(gl[:, -1], gl0[:, -1]) and torch.equal(ga[:, -1], ga0[:, -1])
    assert torch.isnan(gl[:, :-1]).all() and torch.isnan(ga[:, :-1]).all()


def test_empty_queries_with_an_order():
    w = Workload("e", 2, 2, ((5, 6),), 0, 2, 8, 2, "f32", "uniform", 0, (0, 1), 1)
    d = _to_dev(make_inputs(w))
    order = torch.empty((0,), dtype=torch.int32, device=DEV)
    out = msda_forward(d["value"], d["spatial_shapes"], d["level_start_index"],
                       d["sampling_locations"], d["attention_weights"], query_order=order)
    assert out.shape == (2, 0, 16)


@pytest.mark.parametrize("name", ["detr_encoder", "detr_encoder_bf16_b8", "volume3d"])
def test_full_size_workloads_in_the_bench_order(name):
    # the launch configuration the benchmark times: the full workload visited
    # in the interleaved Z-order.  Forward, fused forward and the location and
    # weight gradients bitwise against the raw order; forward rows sampled and
    # grad_value in full against the oracle.
    w = CONFIGS[name]
    dims = w.dims
    inp = make_inputs(w)
    d = _to_dev(inp)
    order = msda_query_order(w.shapes, False, device=DEV)
    fwd = msda_forward if dims == 2 else msda3d_forward
    fused = msda_forward_fused if dims == 2 else msda3d_forward_fused
    bwd = msda_backward if dims == 2 else msda3d_backward
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
            d["attention_weights"])
    _log(f"[order] full size {name}: forward")
    base = fwd(*args)
    got = fwd(*args, query_order=order)
    torch.cuda.synchronize()
    assert torch.equal(got, base)
    rows = torch.randperm(w.queries_per_image, generator=torch.Generator().manual_seed(9))[:48]
    sub = dict(inp, sampling_locations=inp["sampling_locations"][:, rows].contiguous(),
               attention_weights=inp["attention_weights"][:, rows].contiguous())
    assert_parity(got[:, rows.to(DEV)], oracle_fwd(dims, sub))
    _log(f"[order] full size {name}: fused forward")
    fin = _to_dev(make_fused_inputs(w))
    fargs = (fin["value"], fin["spatial_shapes"], fin["level_start_index"],
             fin["reference_points"], fin["sampling_offsets"], fin["attention_logits"])
    fb = fused(*fargs)
    fo = fused(*fargs, query_order=order)
    torch.cuda.synchronize()
    assert torch.equal(fo, fb)
    _log(f"[order] full size {name}: backward")
    grad = make_grad_out(w)
    g = grad.to(DEV)
    _, gl0, ga0 = bwd(*args, g)
    gv, gl, ga = bwd(*args, g, query_order=order)
    torch.cuda.synchronize()
    assert torch.equal(gl, gl0) and torch.equal(ga, ga0)
    check_backward(dims, inp, grad, (gv, gl, ga))
