"""Host logic of the benchmark (CPU): the visit order each run uses, and the
committed counters it reads."""
import pytest

import bench
from scale_deformable_attention_02_amd.workloads import CONFIGS


@pytest.mark.parametrize("op", ["forward", "forward_fused", "backward"])
def test_auto_order_for_pixel_centre_workloads(op):
    for name in ("detr_encoder", "detr_encoder_bf16_b8", "volume3d"):
        assert bench.resolve_query_order("auto", CONFIGS[name], op) == "interleaved"


def test_auto_order_exceptions():
    # the 2D pruned forward runs faster in the raw order; the 3D one does not
    assert bench.resolve_query_order("auto", CONFIGS["detr_encoder"], "forward_pruned") == "none"
    assert bench.resolve_query_order("auto", CONFIGS["volume3d"], "forward_pruned") == "interleaved"
    # queries that are not pixel centres get no order
    assert bench.resolve_query_order("auto", CONFIGS["detr_decoder"], "forward") == "none"
    assert bench.resolve_query_order("auto", CONFIGS["tiny"], "backward") == "none"


def test_explicit_orders():
    enc, dec = CONFIGS["detr_encoder"], CONFIGS["detr_decoder"]
    assert bench.resolve_query_order("none", dec, "forward") == "none"
    assert bench.resolve_query_order("levels", enc, "forward_pruned") == "levels"
    assert bench.resolve_query_order("interleaved", dec, "forward") is None


def test_points_order_is_allowed_for_any_queries():
    for name in ("detr_decoder", "tiny", "detr_encoder", "volume3d"):
        assert bench.resolve_query_order("points", CONFIGS[name], "forward") == "points"


def test_committed_counters_match_the_kernel_sources():
    # roofline.traffic of the headline line comes from profiles/*_counters.json,
    # taken on the kernel sources as they are; a kernel change needs new
    # counters (the bench line reports traffic as null until then)
    interleaved = "z-order, levels interleaved"
    assert bench.counters_for("detr_encoder", "forward", interleaved) is not None
    assert bench.counters_for("volume3d", "forward", interleaved) is not None
    assert bench.counters_for("detr_encoder", "backward", interleaved) is not None
