"""Pins of the oracle's front end (softmax of logits, reference + offset)
against facts fixed by the mathematics, independent of its own code:

* equal logits give A = 1/(L*P) exactly (L*P a power of two), so the result
  is the core oracle's with those weights, bit for bit;
* one dominant logit (the others 1e4 lower: exp underflows to exactly 0)
  makes A one-hot, so a sample at a pixel centre returns that pixel's value
  row exactly;
* two samples: A_0 = (1 + tanh((z_0 - z_1)/2)) / 2, the logistic identity, a
  formula the oracle does not use;
* a common shift of the logits leaves the result unchanged;
* with value = 1 everywhere and every sample strictly inside, the output is
  sum A = 1;
* reference + offset: dyadic pairs whose fp32 sum is exact give the core's
  result at that sum; a non-representable sum is rounded once in fp32, the
  same as torch's fp32 addition.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (msda3d_oracle_forward, msda3d_oracle_forward_fused, msda_oracle_forward,
                    msda_oracle_forward_fused)


def _setup(dims, N=1, Lq=3, M=2, D=4, L=2, P=4, seed=0):
    rng = np.random.default_rng(seed)
    # power-of-two extents: pixel centres (j + 0.5) / W are exact in fp32 and
    # map to x_hat = j exactly
    shapes = [(4, 8), (2, 4)] if dims == 2 else [(2, 4, 8), (2, 2, 4)]
    shapes = shapes[:L]
    sizes = [int(np.prod(s)) for s in shapes]
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    S = int(sum(sizes))
    value = rng.standard_normal((N, S, M, D))
    return (value, np.array(shapes, np.int64), starts, rng, S)


@pytest.mark.parametrize("dims", [2, 3])
def test_equal_logits_give_uniform_weights(dims):
    value, shapes, starts, rng, S = _setup(dims)
    N, Lq, M, L, P = 1, 3, 2, 2, 4
    ref = rng.uniform(0.1, 0.9, (N, Lq, dims)).astype(np.float32)
    off = (rng.standard_normal((N, Lq, M, L, P, dims)) * 0.1).astype(np.float32)
    z = np.full((N, Lq, M, L, P), 0.731)
    out = (msda_oracle_forward_fused if dims == 2 else msda3d_oracle_forward_fused)(
        value, shapes, starts, ref, off, z)
    loc = (ref.reshape(N, Lq, 1, 1, 1, dims) + off).astype(np.float32)
    core = (msda_oracle_forward if dims == 2 else msda3d_oracle_forward)(
        value, shapes, starts, loc, np.full((N, Lq, M, L, P), 1.0 / (L * P)))
    assert np.array_equal(out, core)


@pytest.mark.parametrize("dims", [2, 3])
def test_dominant_logit_is_an_exact_gather(dims):
    value, shapes, starts, rng, S = _setup(dims)
    N, Lq, M, L, P = 1, 4, 2, 2, 4
    ext = shapes[:, ::-1]                  # (W, H[, Z]) per level
    ref = np.zeros((N, Lq, dims), np.float32)
    off = np.zeros((N, Lq, M, L, P, dims), np.float32)
    z = np.full((N, Lq, M, L, P), -1e4)
    expect = np.zeros((N, Lq, M, value.shape[3]))
    for q in range(Lq):
        for m in range(M):
            l, p = rng.integers(0, L), rng.integers(0, P)
            z[0, q, m, l, p] = 0.0
            idx = [int(rng.integers(0, e)) for e in ext[l]]       # (j, i[, k])
            # reference at the level's origin corner, offset to the pixel centre
            for c in range(dims):
                off[0, q, m, l, p, c] = (idx[c] + 0.5) / ext[l][c]
            flat = idx[0] + ext[l][0] * idx[1] + (ext[l][0] * ext[l][1] * idx[2] if dims == 3 else 0)
            expect[0, q, m] = value[0, starts[l] + flat, m]
    out = (msda_oracle_forward_fused if dims == 2 else msda3d_oracle_forward_fused)(
        value, shapes, starts, ref, off, z)
    assert np.array_equal(out.reshape(N, Lq, M, -1), expect)


def test_two_samples_follow_the_logistic_identity():
    value, shapes, starts, rng, S = _setup(2, L=1)
    N, Lq, M, L, P = 1, 5, 2, 1, 2
    H, W = shapes[0]
    ref = np.zeros((N, Lq, 2), np.float32)
    off = np.zeros((N, Lq, M, L, P, 2), np.float32)
    pix = rng.integers(0, [W, H], size=(Lq, M, P, 2))
    off[0, :, :, 0, :, 0] = (pix[..., 0] + 0.5) / W
    off[0, :, :, 0, :, 1] = (pix[..., 1] + 0.5) / H
    z = rng.normal(0, 2, (N, Lq, M, L, P))
    out = msda_oracle_forward_fused(value, shapes, starts, ref, off, z).reshape(Lq, M, -1)
    for q in range(Lq):
        for m in range(M):
            a0 = 0.5 * (1.0 + math.tanh(0.5 * (z[0, q, m, 0, 0] - z[0, q, m, 0, 1])))
            v = [value[0, pix[q, m, k, 0] + W * pix[q, m, k, 1], m] for k in range(2)]
            np.testing.assert_allclose(out[q, m], a0 * v[0] + (1 - a0) * v[1],
                                       rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("dims", [2, 3])
def test_shift_of_the_logits_changes_nothing(dims):
    value, shapes, starts, rng, S = _setup(dims, seed=3)
    N, Lq, M, L, P = 1, 6, 2, 2, 4
    ref = rng.uniform(0, 1, (N, Lq, dims)).astype(np.float32)
    off = (rng.standard_normal((N, Lq, M, L, P, dims)) * 0.2).astype(np.float32)
    z = rng.standard_normal((N, Lq, M, L, P))
    fn = msda_oracle_forward_fused if dims == 2 else msda3d_oracle_forward_fused
    a = fn(value, shapes, starts, ref, off, z)
    b = fn(value, shapes, starts, ref, off, z + 37.0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dims", [2, 3])
def test_weights_sum_to_one(dims):
    value, shapes, starts, rng, S = _setup(dims, seed=4)
    N, Lq, M, L, P = 1, 7, 2, 2, 4
    ones = np.ones_like(value)
    # references and offsets keep every sample strictly inside every level
    ref = rng.uniform(0.4, 0.6, (N, Lq, dims)).astype(np.float32)
    off = rng.uniform(-0.05, 0.05, (N, Lq, M, L, P, dims)).astype(np.float32)
    z = rng.standard_normal((N, Lq, M, L, P)) * 3
    fn = msda_oracle_forward_fused if dims == 2 else msda3d_oracle_forward_fused
    out = fn(ones, shapes, starts, ref, off, z)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_reference_plus_offset():
    value, shapes, starts, rng, S = _setup(2, seed=5)
    N, Lq, M, L, P = 1, 9, 2, 2, 4
    # dyadic reference points and offsets: the fp32 sum is exact
    ref = (rng.integers(0, 64, (N, Lq, 2)) / 64.0).astype(np.float32)
    off = (rng.integers(-16, 17, (N, Lq, M, L, P, 2)) / 256.0).astype(np.float32)
    z = np.zeros((N, Lq, M, L, P))
    exact = ref.astype(np.float64).reshape(N, Lq, 1, 1, 1, 2) + off.astype(np.float64)
    out = msda_oracle_forward_fused(value, shapes, starts, ref, off, z)
    core = msda_oracle_forward(value, shapes, starts, exact.astype(np.float32),
                               np.full((N, Lq, M, L, P), 1.0 / (L * P)))
    assert np.array_equal(out, core)
    # a sum that is not representable is rounded once in fp32 (torch's fp32 add)
    ref2 = np.full((N, Lq, 2), 0.1, np.float32)
    off2 = np.full((N, Lq, M, L, P, 2), 1e-8, np.float32)
    loc2 = (torch.from_numpy(ref2).reshape(N, Lq, 1, 1, 1, 2) + torch.from_numpy(off2)).numpy()
    out2 = msda_oracle_forward_fused(value, shapes, starts, ref2, off2, z)
    core2 = msda_oracle_forward(value, shapes, starts, np.ascontiguousarray(loc2),
                                np.full((N, Lq, M, L, P), 1.0 / (L * P)))
    assert np.array_equal(out2, core2)
