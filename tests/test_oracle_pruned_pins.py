"""Pins of the oracle's pruning rule (DEFA, abstract: sampling points pruned
by their probability; read as: a sample whose attention weight is below the
threshold contributes nothing, the others are unchanged), against facts that
do not go through its code:

* threshold -inf keeps everything: the plain forward, bit for bit;
* a threshold above every weight drops everything: exact zeros;
* one-hot-location samples at pixel centres: the output is the sum of
  A * value row over the kept samples, written out here by hand, and a weight
  equal to the threshold is kept (the test is strict);
* NaN weights are kept (the output turns NaN).
"""
import numpy as np
import pytest

from oracle import (msda3d_oracle_forward, msda3d_oracle_forward_pruned, msda_oracle_forward,
                    msda_oracle_forward_pruned)


def _inputs(dims, seed=0, N=2, Lq=5, M=2, D=4, P=3):
    rng = np.random.default_rng(seed)
    shapes = np.array([(4, 8), (2, 4)] if dims == 2 else [(2, 4, 8), (2, 2, 4)], np.int64)
    sizes = shapes.prod(axis=1)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    S = int(sizes.sum())
    L = len(shapes)
    value = rng.standard_normal((N, S, M, D))
    loc = rng.uniform(-0.1, 1.1, (N, Lq, M, L, P, dims)).astype(np.float32)
    attw = rng.dirichlet(np.ones(L * P), size=(N, Lq, M)).reshape(N, Lq, M, L, P)
    attw = attw.astype(np.float32).astype(np.float64)
    return value, shapes, starts, loc, attw, rng


@pytest.mark.parametrize("dims", [2, 3])
def test_minus_infinity_keeps_everything(dims):
    value, shapes, starts, loc, attw, _ = _inputs(dims)
    fwd = msda_oracle_forward if dims == 2 else msda3d_oracle_forward
    pr = msda_oracle_forward_pruned if dims == 2 else msda3d_oracle_forward_pruned
    assert np.array_equal(pr(value, shapes, starts, loc, attw, -np.inf),
                          fwd(value, shapes, starts, loc, attw))


@pytest.mark.parametrize("dims", [2, 3])
def test_threshold_above_every_weight_gives_zeros(dims):
    value, shapes, starts, loc, attw, _ = _inputs(dims, seed=1)
    pr = msda_oracle_forward_pruned if dims == 2 else msda3d_oracle_forward_pruned
    out = pr(value, shapes, starts, loc, attw, 1.5)
    assert np.count_nonzero(out) == 0


@pytest.mark.parametrize("dims", [2, 3])
def test_kept_samples_at_pixel_centres(dims):
    value, shapes, starts, _, _, rng = _inputs(dims, seed=2)
    N, S, M, D = value.shape
    Lq, L, P = 6, len(shapes), 3
    ext = shapes[:, ::-1]
    loc = np.zeros((N, Lq, M, L, P, dims), np.float32)
    flat = np.zeros((N, Lq, M, L, P), np.int64)
    for l in range(L):
        idx = [rng.integers(0, ext[l][c], size=(N, Lq, M, P)) for c in range(dims)]
        for c in range(dims):
            loc[:, :, :, l, :, c] = (idx[c] + 0.5) / ext[l][c]
        f = idx[0] + ext[l][0] * idx[1]
        if dims == 3:
            f = f + ext[l][0] * ext[l][1] * idx[2]
        flat[:, :, :, l, :] = starts[l] + f
    thr = np.float32(0.25)
    attw = rng.choice(np.array([0.125, 0.25, 0.5, 0.0625], np.float32), size=(N, Lq, M, L, P))
    attw = attw.astype(np.float64)
    pr = msda_oracle_forward_pruned if dims == 2 else msda3d_oracle_forward_pruned
    out = pr(value, shapes, starts, loc, attw, thr).reshape(N, Lq, M, D)
    expect = np.zeros((N, Lq, M, D))
    for n in range(N):
        for q in range(Lq):
            for m in range(M):
                for l in range(L):
                    for p in range(P):
                        a = attw[n, q, m, l, p]
                        if a >= thr:             # equal to the threshold: kept
                            expect[n, q, m] += a * value[n, flat[n, q, m, l, p], m]
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-15)
    assert (attw == thr).any() and (attw < thr).any()


def test_nan_weights_are_kept():
    value, shapes, starts, loc, attw, _ = _inputs(2, seed=3)
    loc = np.full_like(loc, 0.5)
    attw[0, 0, 0, 0, 0] = np.nan
    out = msda_oracle_forward_pruned(value, shapes, starts, loc, attw, 0.9)
    assert np.isnan(out[0, 0, :value.shape[3]]).all()
    assert not np.isnan(out[0, 1:]).any()
