"""f64 chunked (WY / UT-transform) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY.  A second, independent formulation of the
recurrence, used to pin the sequential oracle (the two must agree to rounding)
and to check the chunked algebra before any GPU code uses it.  numpy only; it
imports nothing from the sequential oracle or the GPU path.

Derivation (exact arithmetic).  Write one token's update as
S_t = a_t S_{t-1} + u_t k_t^T with u_t = b_t (v_t - a_t S_{t-1} k_t).  Inside a
chunk of n tokens that starts from S_0, let G_t = sum_{s<=t} log a_s and
gamma_t = e^{G_t}.  Unrolling gives S_t = gamma_t S_0 + sum_{j<=t} e^{G_t-G_j} u_j k_j^T,
and substituting into u_t yields the unit lower-triangular system

    (I + A) U = diag(b) V - diag(b gamma) K S_0^T,
    A_tj = b_t e^{G_t - G_j} (k_t . k_j)   for j < t, 0 otherwise.

With Tm = (I + A)^{-1}, W = Tm diag(b gamma) K and Ut = Tm diag(b) V, and
H = S^T ([dk, dv]):

    U   = Ut - W H_0
    O   = diag(gamma) Q H_0 + (M o Q K^T) U,   M_tj = e^{G_t - G_j} (j <= t)
    H_n = gamma_n H_0 + Kt^T U,                Kt_j = e^{G_n - G_j} k_j

Only non-positive exponents occur (G_t - G_j with j <= t, and G_t itself).
"""
import numpy as np


def chunk_step(q, k, v, g, beta, H0):
    """One chunk for one head.  q, k: [n, dk]; v: [n, dv]; g = log(alpha): [n];
    beta: [n]; H0 = S0^T: [dk, dv].  Returns (o [n, dv], H_n [dk, dv])."""
    n = q.shape[0]
    G = np.cumsum(g)
    gamma = np.exp(G)
    diff = G[:, None] - G[None, :]
    lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower = np.tril(np.ones((n, n), dtype=bool), 0)
    decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    KK = k @ k.T
    A = np.where(lower_strict, beta[:, None] * decay * KK, 0.0)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ ((beta * gamma)[:, None] * k)
    Ut = Tm @ (beta[:, None] * v)
    U = Ut - W @ H0
    P = decay * (q @ k.T)
    o = gamma[:, None] * (q @ H0) + P @ U
    Kt = np.exp(G[-1] - G)[:, None] * k
    Hn = gamma[-1] * H0 + Kt.T @ U
    return o, Hn


def recurrence_chunked(q, k, v, alpha, beta, S0=None, chunk=64, q_scale=1.0):
    """Same contract as ``oracle.recurrence`` (q, k: [B,T,Hk,dk], v: [B,T,Hv,dv],
    alpha, beta: [B,T,Hv], S0: [B,Hv,dv,dk]) computed chunk by chunk; the last
    chunk may be shorter.  Returns (o, S)."""
    q = np.asarray(q, dtype=np.float64) * q_scale
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    group = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    S = np.zeros((B, Hv, dv, dk))
    with np.errstate(divide="ignore"):
        g_all = np.log(alpha)
    for b in range(B):
        for h in range(Hv):
            kh = h // group
            H = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64).T
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                oc, H = chunk_step(q[b, c0:c1, kh], k[b, c0:c1, kh], v[b, c0:c1, h],
                                   g_all[b, c0:c1, h], beta[b, c0:c1, h], H)
                o[b, c0:c1, h] = oc
            S[b, h] = H.T
    return o, S
