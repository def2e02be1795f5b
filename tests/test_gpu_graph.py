"""GPU: the entry points captured in a HIP graph (torch.cuda.CUDAGraph).

The library allocates, synchronises and memsets nothing (the backward clears
grad_value with a fill kernel, not a memset node), so a sequence of calls can
be captured once and replayed.  One graph holds the order builders, the plain,
pruned and fused forwards and the backward of an encoder-shaped pyramid large
enough for the staged forward and the de-duplicating backward, and two value
projections (the tiled and the W-stationary kernel).  It is replayed several
times, with new inputs copied into its tensors between the replays and the
same calls made eagerly
after each replay; every replay is checked against those eager results: bit
for bit where the kernels are deterministic (forwards, order, location and
weight gradients, projection), and grad_value, whose fp32 atomics add in any
order, against the oracle to the backward's bounds.
"""
import pytest
import torch

from scale_deformable_attention_02_amd import (msda_backward, msda_forward, msda_forward_fused,
                                               msda_forward_pruned, msda_linear,
                                               msda_query_order, msda_query_order_points)
from scale_deformable_attention_02_amd.workloads import (Workload, make_fused_inputs,
                                                         make_grad_out, make_inputs,
                                                         make_linear_inputs)
from test_gpu_backward import check_backward

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SHAPES = ((60, 90), (30, 45), (15, 23), (8, 12))
THRESHOLD = 0.8 / 16


def _workload(seed):
    # pixel-centre queries, N = 2, M = 8: 115,056 (query, head) tiles
    return Workload("graph", 2, 2, SHAPES, None, 8, 32, 4, "f32", "pixel_centres", 0.03,
                    (0.0, 1.0), seed)


def _draw(seed):
    w = _workload(seed)
    inp = make_inputs(w)
    fin = make_fused_inputs(w)
    grad = make_grad_out(w)
    # the tiled projection kernel, and (65,573 rows) the W-stationary one
    lin = {"small": make_linear_inputs(64 * 37, 256, 256, "bf16", seed=seed),
           "large": make_linear_inputs(65573, 256, 256, "bf16", seed=seed + 1)}
    return w, inp, fin, grad, lin


class Static:
    """The graph's tensors: inputs are overwritten in place before a replay."""

    def __init__(self, inp, fin, grad, lin):
        self.inp = {k: v.to(DEV) for k, v in inp.items()}
        self.fin = {k: v.to(DEV) for k, v in fin.items()}
        self.grad = grad.to(DEV)
        self.lin = {n: {k: v.to(DEV) for k, v in d.items()} for n, d in lin.items()}
        # the points order follows each query's first sampling location
        self.points = inp["sampling_locations"][0, :, 0, 0, 0, :].contiguous().to(DEV)
        N, Lq, M, L, P, _ = inp["sampling_locations"].shape
        S = inp["value"].shape[1]
        D = inp["value"].shape[3]
        f32 = dict(dtype=torch.float32, device=DEV)
        self.order = torch.empty((S,), dtype=torch.int32, device=DEV)
        self.porder = torch.empty((Lq,), dtype=torch.int32, device=DEV)
        self.out = torch.empty((N, Lq, M * D), **f32)
        self.out_pruned = torch.empty((N, Lq, M * D), **f32)
        self.out_fused = torch.empty((N, Lq, M * D), **f32)
        self.gv = torch.empty(inp["value"].shape, **f32)
        self.gl = torch.empty(inp["sampling_locations"].shape, **f32)
        self.ga = torch.empty(inp["attention_weights"].shape, **f32)
        self.y = torch.empty((lin["small"]["x"].shape[0], lin["small"]["weight"].shape[0]),
                             dtype=torch.bfloat16, device=DEV)
        self.y_large = torch.empty((lin["large"]["x"].shape[0], lin["large"]["weight"].shape[0]),
                                   dtype=torch.bfloat16, device=DEV)

    def load(self, inp, fin, grad, lin):
        for k, v in inp.items():
            self.inp[k].copy_(v)
        for k, v in fin.items():
            self.fin[k].copy_(v)
        self.grad.copy_(grad)
        for n, d in lin.items():
            for k, v in d.items():
                self.lin[n][k].copy_(v)
        self.points.copy_(inp["sampling_locations"][0, :, 0, 0, 0, :])

    def run(self):
        d, f = self.inp, self.fin
        msda_query_order(SHAPES, False, out=self.order)
        msda_query_order_points(self.points, out=self.porder)
        args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
                d["attention_weights"])
        msda_forward(*args, out=self.out, query_order=self.order)
        msda_forward_pruned(*args, THRESHOLD, out=self.out_pruned)
        msda_forward_fused(f["value"], f["spatial_shapes"], f["level_start_index"],
                           f["reference_points"], f["sampling_offsets"], f["attention_logits"],
                           out=self.out_fused, query_order=self.porder)
        msda_backward(*args, self.grad, grad_value=self.gv, grad_sampling_locations=self.gl,
                      grad_attention_weights=self.ga, query_order=self.order)
        for n, y in (("small", self.y), ("large", self.y_large)):
            msda_linear(self.lin[n]["x"], self.lin[n]["weight"], self.lin[n]["bias"], out=y)

    def results(self):
        return {k: getattr(self, k).clone() for k in
                ("order", "porder", "out", "out_pruned", "out_fused", "gv", "gl", "ga", "y",
                 "y_large")}


def test_graph_replays_match_eager_calls():
    _, inp0, fin0, grad0, lin0 = _draw(4100)
    st = Static(inp0, fin0, grad0, lin0)

    # warm up on a side stream (default priority), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()

    eager_state = Static(inp0, fin0, grad0, lin0)
    for r, seed in enumerate((4101, 4102, 4103)):
        _, inp, fin, grad, lin = _draw(seed)
        print(f"[graph] replay {r}: inputs of seed {seed}", flush=True)
        st.load(inp, fin, grad, lin)
        graph.replay()
        torch.cuda.synchronize()
        got = st.results()

        # the same calls, eagerly, on the same inputs
        eager_state.load(inp, fin, grad, lin)
        eager_state.run()
        torch.cuda.synchronize()
        ref = eager_state.results()

        for k in ("order", "porder", "out", "out_pruned", "out_fused", "gl", "ga", "y", "y_large"):
            assert torch.equal(got[k], ref[k]), f"replay {r}: {k} differs from the eager call"

        # grad_value: fp32 atomics add in any order; checked against the oracle
        check_backward(2, inp, grad, (got["gv"], got["gl"], got["ga"]))
