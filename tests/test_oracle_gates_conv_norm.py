"""Pins for the oracle's gates, conv+silu, L2 and gated RMSNorm.

Each test fixes the oracle to something other than itself: a closed form, a
numpy/scipy library routine, or an invariant the definition implies ("Qwen3.8
27B" model card, Gated DeltaNet and Norms bullets; llm-arch-viz module tree).
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle

# ---------------------------------------------------------------- gates


def test_gates_closed_forms():
    # a + dt_bias = 0 and A_log = 0: g = -softplus(0) = -ln 2, alpha = 1/2; b = 0: beta = 1/2.
    alpha, beta, g = oracle.gates(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros(2), np.zeros(2))
    assert np.allclose(alpha, 0.5, rtol=0, atol=1e-16)
    assert np.all(beta == 0.5)
    assert np.allclose(g, -np.log(2.0), rtol=0, atol=1e-16)
    # a and dt_bias enter only through their sum.
    a1, _, _ = oracle.gates(np.array([[0.3]]), np.zeros((1, 1)), np.zeros(1), np.array([-0.3]))
    assert abs(a1[0, 0] - 0.5) < 1e-15


def test_gates_infinities():
    inf = np.inf
    # beta: b = -inf -> 0, b = +inf -> 1 exactly.
    _, beta, _ = oracle.gates(np.zeros((1, 2)), np.array([[-inf, inf]]), np.zeros(2), np.zeros(2))
    assert beta[0, 0] == 0.0 and beta[0, 1] == 1.0
    # alpha: a = -inf -> softplus 0 -> alpha 1; a = +inf -> alpha 0; A_log = -inf -> alpha 1.
    alpha, _, _ = oracle.gates(np.array([[-inf, inf, 5.0]]), np.zeros((1, 3)),
                               np.array([0.0, 0.0, -inf]), np.zeros(3))
    assert alpha[0, 0] == 1.0 and alpha[0, 1] == 0.0 and alpha[0, 2] == 1.0


def test_gates_against_library_routines():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 3, 500), [-40.0, -20.0, 20.0, 40.0, 700.0, -700.0]])
    H = x.size
    a = x[None, :]
    alpha, beta, g = oracle.gates(a, a, np.zeros(H), np.zeros(H))
    # With A_log = 0: -g is softplus(a) = log(1 + e^a) = logaddexp(0, a).
    assert np.allclose(-g[0], np.logaddexp(0.0, x), rtol=1e-15, atol=0)
    assert np.allclose(beta[0], expit(x), rtol=1e-15, atol=1e-300)
    # A_log scales the log-decay by exp(A_log): doubling via A_log = ln 2.
    _, _, g2 = oracle.gates(a, a, np.full(H, np.log(2.0)), np.zeros(H))
    assert np.allclose(g2, 2.0 * g, rtol=1e-15, atol=0)
    # Decay is monotone: larger a -> smaller alpha.
    order = np.argsort(x)
    assert np.all(np.diff(alpha[0][order]) <= 0)


# ---------------------------------------------------------------- conv + silu

def _silu(x):
    return x * expit(x)


def test_conv_identity_tap_is_silu():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(2, 9, 5))
    w = np.zeros((5, 4))
    w[:, 3] = 1.0  # the last tap multiplies the current token
    y, hist = oracle.conv_silu(x, w)
    assert np.allclose(y, _silu(x), rtol=1e-15, atol=1e-300)
    assert np.array_equal(hist, x[:, -3:, :])


def test_conv_impulse_reads_taps_in_order():
    rng = np.random.default_rng(2)
    C, T, t0 = 3, 10, 4
    w = rng.normal(size=(C, 4))
    x = np.zeros((1, T, C))
    x[0, t0, :] = 1.0
    y, _ = oracle.conv_silu(x, w)
    for c in range(C):
        for t in range(T):
            lag = t - t0
            pre = w[c, 3 - lag] if 0 <= lag <= 3 else 0.0
            assert abs(y[0, t, c] - _silu(pre)) < 1e-15


def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(3)
    B, T, C = 2, 17, 6
    x = rng.normal(size=(B, T, C))
    w = rng.normal(size=(C, 4))
    hist = rng.normal(size=(B, 3, C))
    y, hist_out = oracle.conv_silu(x, w, hist)
    for b in range(B):
        for c in range(C):
            xhat = np.concatenate([hist[b, :, c], x[b, :, c]])
            pre = np.convolve(xhat, w[c, ::-1], mode="valid")
            assert np.allclose(y[b, :, c], _silu(pre), rtol=1e-13, atol=1e-15)
            assert np.array_equal(hist_out[b, :, c], xhat[-3:])


def test_conv_split_with_history_is_bitwise_equal():
    rng = np.random.default_rng(4)
    B, T, C = 2, 23, 7
    x = rng.normal(size=(B, T, C))
    w = rng.normal(size=(C, 4))
    y_full, h_full = oracle.conv_silu(x, w)
    for t1 in (1, 2, 3, 11):
        y1, h1 = oracle.conv_silu(x[:, :t1], w)
        y2, h2 = oracle.conv_silu(x[:, t1:], w, h1)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y_full)
        assert np.array_equal(h2, h_full)


def test_conv_short_sequence_history_shift():
    # T < W-1: the new history is the tail of [old history; x].
    rng = np.random.default_rng(5)
    x = rng.normal(size=(1, 2, 4))
    hist = rng.normal(size=(1, 3, 4))
    _, h = oracle.conv_silu(x, rng.normal(size=(4, 4)), hist)
    assert np.array_equal(h[0], np.concatenate([hist[0, 2:], x[0]]))


# ---------------------------------------------------------------- L2

def test_l2_unit_norm_and_library():
    rng = np.random.default_rng(6)
    y = rng.normal(size=(5, 3 * 8 + 4))
    out = oracle.l2norm_heads(y, 3 * 8, 8, eps=1e-6)
    for g in range(3):
        seg = y[:, g * 8:(g + 1) * 8]
        ref = seg / np.sqrt(np.linalg.norm(seg, axis=1, keepdims=True) ** 2 + 1e-6)
        assert np.allclose(out[:, g * 8:(g + 1) * 8], ref, rtol=1e-14, atol=0)
    assert np.allclose(np.linalg.norm(out[:, :24].reshape(5, 3, 8), axis=2), 1.0, atol=1e-6)
    assert np.array_equal(out[:, 24:], y[:, 24:])  # channels past l2_channels untouched


def test_l2_constant_and_zero_vectors():
    D, c, eps = 128, -0.37, 1e-6
    y = np.full((1, D), c)
    out = oracle.l2norm_heads(y, D, D, eps)
    assert np.allclose(out, c / np.sqrt(D * c * c + eps), rtol=1e-15)
    z = oracle.l2norm_heads(np.zeros((1, D)), D, D, eps)
    assert np.all(z == 0.0)


# ---------------------------------------------------------------- gated RMSNorm

def test_gated_rmsnorm_closed_forms():
    D, eps = 128, 1e-6
    c = 0.8
    x = np.full((1, 1, D), c)
    z = np.full((1, 1, D), 1.3)
    w = np.linspace(-0.5, 0.5, D)
    y = oracle.gated_rmsnorm(x, z, w, eps)
    expect = c / np.sqrt(c * c + eps) * (1 + w) * _silu(1.3)
    assert np.allclose(y[0, 0], expect, rtol=1e-15)
    # Alternating signs: RMS is 1 (mean, not sum, of squares).
    xs = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)[None, None, :]
    y2 = oracle.gated_rmsnorm(xs, z, np.zeros(D), eps)
    assert np.allclose(y2[0, 0], xs[0, 0] / np.sqrt(1 + eps) * _silu(1.3), rtol=1e-15)


def test_gated_rmsnorm_zeros_and_invariance():
    rng = np.random.default_rng(8)
    N, H, D = 3, 4, 16
    x = rng.normal(size=(N, H, D))
    z = rng.normal(size=(N, H, D))
    w = rng.normal(0, 0.1, D)
    assert np.all(oracle.gated_rmsnorm(x, np.zeros_like(z), w) == 0.0)
    assert np.all(oracle.gated_rmsnorm(x, z, -np.ones(D)) == 0.0)
    # eps = 0: the normalised part is invariant to scaling each head.
    y0 = oracle.gated_rmsnorm(x, z, w, eps=0.0)
    y1 = oracle.gated_rmsnorm(7.5 * x, z, w, eps=0.0)
    assert np.allclose(y0, y1, rtol=1e-14, atol=1e-15)
    # Per-head: RMS of x*r over D equals 1 when w = 0 and silu(z) = 1 is factored out.
    y = oracle.gated_rmsnorm(x, z, np.zeros(D), eps=0.0) / _silu(z)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    # Heads are independent: permuting heads permutes outputs.
    perm = np.array([2, 0, 3, 1])
    yp = oracle.gated_rmsnorm(x[:, perm], z[:, perm], w)
    assert np.array_equal(yp, oracle.gated_rmsnorm(x, z, w)[:, perm])


def test_mixer_composes_parts():
    # The whole-path helper is exactly its parts in the card's order.
    rng = np.random.default_rng(9)
    B, T, Hk, Hv, d = 1, 6, 1, 2, 4
    C = 2 * Hk * d + Hv * d
    qkv = rng.normal(size=(B, T, C))
    w = rng.normal(0, 0.5, (C, 4))
    z = rng.normal(size=(B, T, Hv * d))
    a = rng.normal(size=(B, T, Hv))
    b = rng.normal(size=(B, T, Hv))
    A_log = rng.uniform(-1, 1, Hv)
    dtb = rng.normal(0, 0.1, Hv)
    nw = rng.normal(0, 0.1, d)
    y, S, h = oracle.mixer(qkv, w, z, a, b, A_log, dtb, nw, Hk, Hv, d)
    yc, hc = oracle.conv_silu(qkv, w)
    yc = oracle.l2norm_heads(yc.reshape(T, C), 2 * Hk * d, d).reshape(B, T, C)
    al, be, _ = oracle.gates(a, b, A_log, dtb)
    o, S2 = oracle.recurrence(yc[:, :, :d].reshape(B, T, 1, d), yc[:, :, d:2 * d].reshape(B, T, 1, d),
                              yc[:, :, 2 * d:].reshape(B, T, Hv, d), al, be)
    y2 = oracle.gated_rmsnorm(o, z.reshape(B, T, Hv, d), nw).reshape(B, T, Hv * d)
    assert np.array_equal(y, y2) and np.array_equal(S, S2) and np.array_equal(h, hc)
