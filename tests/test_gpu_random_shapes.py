"""GPU parity over a seeded random sweep of problem shapes.

Each case draws the dimensionality (2D/3D), the number of levels and their
sizes (down to 1 pixel wide), heads, channels (any multiple of 16 bytes of
value up to 64 channels), points per level (L*P <= 64), queries and batch,
the value and output dtypes, the query layout and the query visit order (none,
a random permutation, or the points order), and a few cases large enough for
the forward's LDS-staged kernel.  Every case runs the forward, the pruned and
fused forwards and the backward, each against the oracle to the tolerance of
its own parity test (same bounds, same helpers).
"""
import numpy as np
import pytest
import torch

from scale_deformable_attention_02_amd import (msda3d_forward, msda3d_forward_fused,
                                               msda3d_forward_pruned, msda_forward,
                                               msda_forward_fused, msda_forward_pruned,
                                               msda_query_order_points)
from scale_deformable_attention_02_amd.workloads import (Workload, make_fused_inputs,
                                                         make_grad_out, make_inputs)
from test_gpu_backward import check_backward, gpu_bwd
from test_gpu_fused import check as check_fused
from test_gpu_parity import assert_parity, oracle_fwd
from test_gpu_pruned import check as check_pruned

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SWEEP_SEED = 20261203
N_CASES = 36
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw_cases(n=N_CASES, seed=SWEEP_SEED):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dims = 3 if i % 3 == 2 else 2
        large = i % 9 in (4, 8)
        L = int(rng.integers(1, 6))
        hi = 48 if dims == 2 else 12
        shapes = tuple(tuple(int(rng.integers(1, hi + 1)) for _ in range(dims))
                       for _ in range(L))
        vdt = "bf16" if rng.random() < 0.35 else "f32"
        per16 = 4 if vdt == "f32" else 8              # channels per 16 bytes
        D = per16 * int(rng.integers(1, 64 // per16 + 1))
        M = int(rng.choice([1, 2, 3, 4, 8]))
        P = int(rng.integers(1, min(8, 64 // L) + 1))
        if large:
            M = 8
            Lq = int(rng.integers(8200, 12000))
            N = 1
        else:
            Lq = int(rng.integers(1, 500))
            N = int(rng.integers(1, 4))
        odt = "bf16" if rng.random() < 0.3 else "f32"
        layout = str(rng.choice(["uniform", "random_refs"]))
        order = str(rng.choice(["none", "random", "points"]))
        cases.append((i, dims, vdt, odt, N, shapes, Lq, M, D, P, layout, order))
    return cases


CASES = _draw_cases()


def _case_id(c):
    i, dims, vdt, odt, N, shapes, Lq, M, D, P, layout, order = c
    return f"{i}-{dims}d-{vdt}>{odt}-N{N}-L{len(shapes)}-Lq{Lq}-M{M}-D{D}-P{P}-{layout}-{order}"


def _order(kind, inp, Lq, seed):
    if kind == "none":
        return None
    if kind == "random":
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        return torch.randperm(Lq, generator=g).to(torch.int32).to(DEV)
    pts = inp["sampling_locations"][0, :, 0, 0, 0, :].contiguous().to(DEV)
    return msda_query_order_points(pts)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_random_shape(case):
    i, dims, vdt, odt, N, shapes, Lq, M, D, P, layout, order = case
    print(f"[random] {_case_id(case)} shapes={shapes}", flush=True)
    w = Workload("random", dims, N, shapes, Lq, M, D, P, vdt, layout,
                 0.1 if layout == "random_refs" else 0.0, (-0.2, 1.2), SWEEP_SEED + i)
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    qo = _order(order, inp, Lq, SWEEP_SEED + i)

    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"])
    kw = dict(out_dtype=TORCH_DT[odt], query_order=qo)

    # forward
    fwd = msda_forward if dims == 2 else msda3d_forward
    out = fwd(*args, d["attention_weights"], **kw)
    torch.cuda.synchronize()
    assert_parity(out, oracle_fwd(dims, inp))

    # pruned forward: a threshold near the mean weight 1/(L*P)
    thr = float(np.float32(np.random.default_rng(SWEEP_SEED + i).uniform(0.5, 1.5)
                           / (len(shapes) * P)))
    pruned = msda_forward_pruned if dims == 2 else msda3d_forward_pruned
    pr = pruned(*args, d["attention_weights"], thr, **kw)
    torch.cuda.synchronize()
    check_pruned(dims, inp, thr, pr)
    attw = d["attention_weights"]
    zeroed = torch.where(attw < thr, torch.zeros_like(attw), attw)
    assert torch.equal(pr, fwd(*args, zeroed, **kw))

    # fused forward (its own draws: reference points + offsets, logits)
    finp = make_fused_inputs(w)
    fd = {k: v.to(DEV) for k, v in finp.items()}
    fn = msda_forward_fused if dims == 2 else msda3d_forward_fused
    fo = fn(fd["value"], fd["spatial_shapes"], fd["level_start_index"], fd["reference_points"],
            fd["sampling_offsets"], fd["attention_logits"], **kw)
    torch.cuda.synchronize()
    check_fused(dims, finp, fo)

    # backward
    grad = make_grad_out(w)
    gpu = gpu_bwd(dims, d, grad.to(DEV), query_order=qo)
    check_backward(dims, inp, grad, gpu)

