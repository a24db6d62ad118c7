"""Pins for the oracle's gated delta rule.

The update is the card's gated delta rule written out,
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t ("Qwen3.8 27B"
model card, Gated DeltaNet bullet).  The oracle evaluates it in the expanded
u = S k form; these tests pin it to an exact-rational brute force of the matrix
form, a hand-worked example, closed forms, invariants and the independent
chunked (WY) form.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute, chunk_ref
from synth import recurrence_inputs, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(q, k, v, alpha, beta, S0=None, q_scale=1.0):
    return oracle.recurrence(q, k, v, alpha, beta, S0, q_scale)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "recurrence_d2_t2.json")))
    inp = {n: np.array([[float(Fraction(x)) for x in r] for r in g["inputs"][n]])
           for n in ("k", "v", "q")}
    al = np.array([float(Fraction(x)) for x in g["inputs"]["alpha"]])
    be = np.array([float(Fraction(x)) for x in g["inputs"]["beta"]])
    o, S = _run(inp["q"][None, :, None, :], inp["k"][None, :, None, :], inp["v"][None, :, None, :],
                al[None, :, None], be[None, :, None])
    o_exp = np.array([[float(Fraction(x)) for x in r] for r in g["expected"]["o"]])
    S_exp = np.array([[float(Fraction(x)) for x in r] for r in g["expected"]["S"]])
    assert np.allclose(o[0, :, 0, :], o_exp, rtol=0, atol=1e-15)
    assert np.allclose(S[0, 0], S_exp, rtol=0, atol=1e-15)
    # The brute force reproduces the same fractions exactly.
    ob, Sb = brute.recurrence_exact(
        [[Fraction(x) for x in r] for r in g["inputs"]["q"]],
        [[Fraction(x) for x in r] for r in g["inputs"]["k"]],
        [[Fraction(x) for x in r] for r in g["inputs"]["v"]],
        [Fraction(x) for x in g["inputs"]["alpha"]], [Fraction(x) for x in g["inputs"]["beta"]])
    assert [[str(x) for x in r] for r in ob] == g["expected"]["o"]
    assert [[str(x) for x in r] for r in Sb] == g["expected"]["S"]


def _rand_frac(rng, n, den=8):
    return [Fraction(int(rng.integers(-2 * den, 2 * den + 1)), den) for _ in range(n)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    T, dk, dv = 5, 3, 4
    q = [_rand_frac(rng, dk) for _ in range(T)]
    k = [_rand_frac(rng, dk, 4) for _ in range(T)]
    v = [_rand_frac(rng, dv) for _ in range(T)]
    alpha = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S0 = [_rand_frac(rng, dk) for _ in range(dv)]
    ob, Sb = brute.recurrence_exact(q, k, v, alpha, beta, S0)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    o, S = _run(f(q)[None, :, None, :], f(k)[None, :, None, :], f(v)[None, :, None, :],
                np.array([float(x) for x in alpha])[None, :, None],
                np.array([float(x) for x in beta])[None, :, None], f(S0)[None, None])
    assert np.allclose(o[0, :, 0, :], f(ob), rtol=1e-13, atol=1e-13)
    assert np.allclose(S[0, 0], f(Sb), rtol=1e-13, atol=1e-13)


def test_brute_force_head_sharing():
    # 2 q/k heads, 6 value heads: value head h reads q/k head h // 3.
    rng = np.random.default_rng(11)
    T, d, Hk, Hv = 4, 2, 2, 6
    q = [[_rand_frac(rng, d) for _ in range(Hk)] for _ in range(T)]
    k = [[_rand_frac(rng, d, 4) for _ in range(Hk)] for _ in range(T)]
    v = [[_rand_frac(rng, d) for _ in range(Hv)] for _ in range(T)]
    alpha = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(Hv)] for _ in range(T)]
    beta = [[Fraction(int(rng.integers(0, 9)), 8) for _ in range(Hv)] for _ in range(T)]
    f = lambda x: np.array(x, dtype=object).astype(np.float64)
    o, S = _run(f(q)[None], f(k)[None], f(v)[None], f(alpha)[None], f(beta)[None])
    for h in range(Hv):
        kh = h // 3
        ob, Sb = brute.recurrence_exact([q[t][kh] for t in range(T)], [k[t][kh] for t in range(T)],
                                        [v[t][h] for t in range(T)], [alpha[t][h] for t in range(T)],
                                        [beta[t][h] for t in range(T)])
        assert np.allclose(o[0, :, h, :], f(ob), rtol=1e-13, atol=1e-13)
        assert np.allclose(S[0, h], f(Sb), rtol=1e-13, atol=1e-13)


def test_beta_zero_only_decays():
    x = recurrence_inputs(1, 9, Hk=2, Hv=4, d=8, seed=3, state_std=1.0)
    q, k, v = (to_f64(x[n]) for n in "qkv")
    S0 = to_f64(x["state"])
    alpha = np.random.default_rng(0).uniform(0.2, 1.0, (1, 9, 4))
    o, S = _run(q, k, v, alpha, np.zeros_like(alpha), S0)
    gamma = np.cumprod(alpha, axis=1)
    assert np.allclose(S, gamma[0, -1][None, :, None, None] * S0, rtol=1e-14, atol=0)
    for t in range(9):
        for h in range(4):
            ref = gamma[0, t, h] * S0[0, h] @ q[0, t, h // 2]
            assert np.allclose(o[0, t, h], ref, rtol=1e-13, atol=1e-15)


def test_unit_basis_key_writes_column_exactly():
    # alpha = beta = 1, k = e_j: column j of S becomes v exactly, others unchanged;
    # q = e_j reads it straight back (o_t sees token t's write).
    rng = np.random.default_rng(4)
    d, j = 8, 5
    S0 = rng.normal(size=(1, 1, d, d)).astype(np.float32).astype(np.float64)
    k = np.zeros((1, 1, 1, d)); k[..., j] = 1.0
    v = rng.normal(size=(1, 1, 1, d)).astype(np.float32).astype(np.float64)
    one = np.ones((1, 1, 1))
    o, S = _run(k, k, v, one, one, S0)
    assert np.array_equal(S[0, 0][:, j], v[0, 0, 0])
    keep = [c for c in range(d) if c != j]
    assert np.array_equal(S[0, 0][:, keep], S0[0, 0][:, keep])
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])


def test_unit_key_makes_S_k_equal_v():
    rng = np.random.default_rng(5)
    d = 16
    k = rng.normal(size=d); k /= np.linalg.norm(k)
    v = rng.normal(size=d)
    S0 = rng.normal(size=(1, 1, d, d))
    one = np.ones((1, 1, 1))
    _, S = _run(k[None, None, None], k[None, None, None], v[None, None, None], one, one, S0)
    assert np.allclose(S[0, 0] @ k, v, rtol=0, atol=1e-13)


def test_scalar_ema_closed_form():
    # d = 1, k = +-1: S_t = alpha_t (1 - beta_t) S_{t-1} + beta_t v_t k_t, so
    # S_T = P_{0..T} S_0 + sum_t P_{t+1..T} beta_t v_t k_t with P the product of alpha(1-beta).
    rng = np.random.default_rng(6)
    T = 12
    k = rng.choice([-1.0, 1.0], T)
    v = rng.normal(size=T)
    q = rng.normal(size=T)
    al = rng.uniform(0.1, 1.0, T)
    be = rng.uniform(0.0, 1.0, T)
    s0 = 0.7
    o, S = _run(q[None, :, None, None], k[None, :, None, None], v[None, :, None, None],
                al[None, :, None], be[None, :, None], np.array([[[[s0]]]]))
    f = al * (1 - be)
    for t in range(T):
        st = np.prod(f[:t + 1]) * s0 + sum(np.prod(f[j + 1:t + 1]) * be[j] * v[j] * k[j]
                                           for j in range(t + 1))
        assert abs(o[0, t, 0, 0] - st * q[t]) < 1e-13
    assert abs(S[0, 0, 0, 0] - (np.prod(f) * s0 + sum(np.prod(f[j + 1:]) * be[j] * v[j] * k[j]
                                                       for j in range(T)))) < 1e-13


def test_orthonormal_keys_masked_matmul():
    # Orthonormal keys and S0 = 0: no key interferes, u_t = beta_t v_t, so
    # O = (M o Q K^T) diag(beta) V with M_tj = gamma_t / gamma_j for j <= t.
    rng = np.random.default_rng(7)
    T, d = 48, 64
    K = np.linalg.qr(rng.normal(size=(d, d)))[0][:T]
    Q = rng.normal(size=(T, d))
    V = rng.normal(size=(T, d))
    al = rng.uniform(0.5, 1.0, T)
    be = rng.uniform(0.0, 1.0, T)
    o, _ = _run(Q[None, :, None], K[None, :, None], V[None, :, None], al[None, :, None],
                be[None, :, None])
    G = np.cumsum(np.log(al))
    M = np.tril(np.exp(G[:, None] - G[None, :]))
    ref = (M * (Q @ K.T)) @ (be[:, None] * V)
    assert np.allclose(o[0, :, 0], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_homogeneity_and_q_scale():
    x = recurrence_inputs(1, 20, Hk=2, Hv=4, d=8, seed=8, state_std=0.3)
    q, k, v = (to_f64(x[n]) for n in "qkv")
    alpha, beta, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    S0 = to_f64(x["state"])
    o, S = _run(q, k, v, alpha, beta, S0)
    o2, S2 = _run(q, k, 3.0 * v, alpha, beta, 3.0 * S0)
    assert np.allclose(o2, 3.0 * o, rtol=1e-13, atol=1e-14)
    assert np.allclose(S2, 3.0 * S, rtol=1e-13, atol=1e-14)
    o3, S3 = _run(q, k, v, alpha, beta, S0, q_scale=0.25)
    assert np.allclose(o3, 0.25 * o, rtol=1e-14, atol=1e-16)
    assert np.array_equal(S3, S)


def test_split_invariance_bitwise():
    x = recurrence_inputs(2, 30, Hk=2, Hv=6, d=8, seed=9, state_std=0.1)
    q, k, v = (to_f64(x[n]) for n in "qkv")
    alpha, beta, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    S0 = to_f64(x["state"])
    o, S = _run(q, k, v, alpha, beta, S0)
    t1 = 13
    o1, S1 = _run(q[:, :t1], k[:, :t1], v[:, :t1], alpha[:, :t1], beta[:, :t1], S0)
    o2, S2 = _run(q[:, t1:], k[:, t1:], v[:, t1:], alpha[:, t1:], beta[:, t1:], S1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(S2, S)


def test_contraction_bound():
    rng = np.random.default_rng(10)
    d, T = 8, 25
    k = rng.normal(size=(T, d)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(T, d))
    al = rng.uniform(0.1, 1.0, T)
    be = rng.uniform(0.0, 1.0, T)
    S = rng.normal(size=(d, d))
    for t in range(T):
        _, Sn = _run(k[None, t:t + 1, None], k[None, t:t + 1, None], v[None, t:t + 1, None],
                     al[None, t:t + 1, None], be[None, t:t + 1, None], S[None, None])
        Sn = Sn[0, 0]
        assert np.linalg.norm(Sn) <= al[t] * np.linalg.norm(S) + be[t] * np.linalg.norm(v[t]) + 1e-12
        S = Sn


@pytest.mark.parametrize("T,chunk,A_lo,A_hi,state", [
    (150, 64, -1.0, 1.0, 0.05),     # config-like decay, ragged tail
    (150, 64, -6.0, -4.0, 0.5),      # slow decay: the carry-in matters
    (64, 16, -1.0, 1.0, None),
    (7, 64, -1.0, 1.0, 0.2),         # one short chunk
])
def test_chunked_form_matches_sequential(T, chunk, A_lo, A_hi, state):
    x = recurrence_inputs(1, T, Hk=2, Hv=6, d=16, seed=T + chunk, state_std=state,
                          A_log_range=(A_lo, A_hi))
    q, k, v = (to_f64(x[n]) for n in "qkv")
    alpha, beta, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    S0 = None if state is None else to_f64(x["state"])
    o, S = _run(q, k, v, alpha, beta, S0)
    oc, Sc = chunk_ref.recurrence_chunked(q, k, v, alpha, beta, S0, chunk=chunk)
    assert np.max(np.abs(oc - o)) <= 1e-12 * np.max(np.abs(o))
    assert np.max(np.abs(Sc - S)) <= 1e-12 * np.max(np.abs(S))
