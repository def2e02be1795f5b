"""Pins of the projection oracle (fp64 y = x W^T + b) independent of the
matmul routine it calls: a pure-Python triple loop on small integer inputs
(exact), the identity weight, and a rank-one closed form."""
import numpy as np

from oracle import linear_oracle


def test_matches_a_triple_loop_on_integers():
    rng = np.random.default_rng(0)
    R, K, N = 5, 7, 3
    x = rng.integers(-9, 10, (R, K)).astype(np.float32)
    w = rng.integers(-9, 10, (N, K)).astype(np.float32)
    b = rng.integers(-5, 6, N).astype(np.float32)
    y = linear_oracle(x, w, b)
    for r in range(R):
        for n in range(N):
            acc = int(b[n])
            for k in range(K):
                acc += int(x[r, k]) * int(w[n, k])
            assert y[r, n] == acc


def test_identity_weight_and_no_bias():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 8)).astype(np.float32)
    b = rng.standard_normal(8).astype(np.float32)
    eye = np.eye(8, dtype=np.float32)
    assert np.array_equal(linear_oracle(x, eye, b), x.astype(np.float64) + b.astype(np.float64))
    assert np.array_equal(linear_oracle(x, eye), x.astype(np.float64))


def test_rank_one_closed_form():
    # x[r, k] = u_r, W[n, k] = v_n * 2^-k (dyadic): y = u_r v_n (2 - 2^(1-K))
    K = 12
    u = np.array([1.5, -2.0, 0.25], np.float32)
    v = np.array([3.0, -0.5], np.float32)
    x = np.repeat(u[:, None], K, axis=1)
    w = (v[:, None] * (2.0 ** -np.arange(K))[None, :]).astype(np.float32)
    expect = np.outer(u, v).astype(np.float64) * (2.0 - 2.0 ** (1 - K))
    assert np.array_equal(linear_oracle(x, w), expect)
