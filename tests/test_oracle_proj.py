"""Pins of the oracle's linear map (the projections around the mixer).

y = x W^T with W in the Linear layout [out][in] ("Qwen/Qwen3.8-27B" architecture
viewer, module tree: in_proj_qkv 5120->10240, in_proj_z 5120->6144, in_proj_a /
in_proj_b 5120->48, out_proj 6144->5120).  The pins are chosen so that a
transposed operand, a wrong row stride or a dropped term fails one of them:
rectangular shapes throughout, exact integer sums checked against Python's own
integer arithmetic, identity and permutation weights, numpy's matmul, and
linearity in x and in W.
"""
import numpy as np
import pytest

import oracle


def test_linear_exact_small_integers_brute_force():
    # Integers in [-8, 8]: every product and partial sum is exact in f64, so the
    # result must equal Python's integer arithmetic bit for bit.
    rng = np.random.default_rng(11)
    M, N, K = 5, 7, 13
    x = rng.integers(-8, 9, size=(M, K))
    W = rng.integers(-8, 9, size=(N, K))
    y = oracle.linear(x.astype(np.float64), W.astype(np.float64))
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            assert y[m, n] == sum(int(x[m, k]) * int(W[n, k]) for k in range(K))


def test_linear_matches_numpy_matmul():
    rng = np.random.default_rng(12)
    for (M, N, K) in [(1, 48, 5120), (33, 96, 257), (64, 17, 8)]:
        x = rng.standard_normal((M, K))
        W = rng.standard_normal((N, K)) / np.sqrt(K)
        y = oracle.linear(x, W)
        ref = x @ W.T
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_linear_identity_and_permutation_weights():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((9, 24))
    np.testing.assert_array_equal(oracle.linear(x, np.eye(24)), x)
    perm = rng.permutation(24)[:10]
    P = np.zeros((10, 24))
    P[np.arange(10), perm] = 1.0
    # Row n of W picks input column perm[n].
    np.testing.assert_array_equal(oracle.linear(x, P), x[:, perm])


def test_linear_is_linear_in_x_and_W():
    rng = np.random.default_rng(14)
    x1, x2 = rng.standard_normal((2, 6, 40))
    W1, W2 = rng.standard_normal((2, 11, 40))
    np.testing.assert_allclose(oracle.linear(2.0 * x1 - x2, W1),
                               2.0 * oracle.linear(x1, W1) - oracle.linear(x2, W1),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.linear(x1, W1 + 3.0 * W2),
                               oracle.linear(x1, W1) + 3.0 * oracle.linear(x1, W2),
                               rtol=1e-12, atol=1e-11)


def test_linear_leading_dims_and_empty():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((2, 3, 16))
    W = rng.standard_normal((5, 16))
    y = oracle.linear(x, W)
    assert y.shape == (2, 3, 5)
    np.testing.assert_allclose(y.reshape(6, 5), oracle.linear(x.reshape(6, 16), W), rtol=0, atol=0)
    assert oracle.linear(np.zeros((0, 16)), W).shape == (0, 5)
