"""f64 CPU oracle for the Gated DeltaNet mixer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The GPU library and its Python
binding never import it, and the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain sequential C, f64); this module
only converts numpy arrays to contiguous f64 and calls it.  Each wrapper names
the passage it follows:

* "Qwen3.8 27B" model card, "Gated DeltaNet" bullet -- conv width 4 + silu,
  L2-normalised q/k, decay exp(-exp(A_log)*softplus(a+dt_bias)), write rate
  sigmoid(b), gated delta rule on a [128,128] state per value head, outputs
  RMS-normalised and gated by silu(z); "Norms" bullet -- scale 1+w, f32.
* llm-arch-viz "Qwen/Qwen3.8-27B" module tree -- conv1d 10240x1x4 without bias,
  RMSNormGated width 128, eps 1e-06; the projections in_proj_qkv 5120->10240,
  in_proj_z 5120->6144, in_proj_a / in_proj_b 5120->48 and out_proj 6144->5120,
  each the linear map x W^T.
* The update rule written out: S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
  o_t = S_t q_t.

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
(closed forms, library routines, exact-rational brute force, invariants and the
independent chunked form in ``oracle/chunk_ref.py``).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.gdn_oracle_gates.argtypes = [_D, _D, _D, _D, _D, _D, _D, i64, i32]
        lib.gdn_oracle_conv_silu.argtypes = [_D, _D, _D, _D, _D, i32, i32, i32, i32]
        lib.gdn_oracle_l2norm_heads.argtypes = [_D, i64, i32, i32, i32, dbl]
        lib.gdn_oracle_recurrence.argtypes = [_D, _D, _D, _D, _D, _D, _D, _D,
                                              i32, i32, i32, i32, i32, i32, dbl]
        lib.gdn_oracle_gated_rmsnorm.argtypes = [_D, _D, _D, _D, i64, i32, i32, dbl]
        lib.gdn_oracle_linear.argtypes = [_D, _D, _D, i64, i32, i32]
        lib.gdn_oracle_num_threads.restype = ctypes.c_int
        lib.gdn_oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.gdn_oracle_set_num_threads.restype = None
        for f in ("gdn_oracle_gates", "gdn_oracle_conv_silu", "gdn_oracle_l2norm_heads",
                  "gdn_oracle_recurrence", "gdn_oracle_gated_rmsnorm", "gdn_oracle_linear"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    return None if x is None else x.ctypes.data_as(_D)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().gdn_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops (parallel over independent
    sequences only; the arithmetic does not depend on it)."""
    _load().gdn_oracle_set_num_threads(int(n))


def gates(a, b, A_log, dt_bias):
    """alpha = exp(-exp(A_log)*softplus(a+dt_bias)), beta = sigmoid(b)
    ("Qwen3.8 27B" card, Gated DeltaNet bullet).  a, b: [..., H]; A_log,
    dt_bias: [H].  Returns (alpha, beta, g) with g = log(alpha)."""
    a = _f64(a)
    b = _f64(b)
    H = a.shape[-1]
    N = a.size // H
    A_log = _f64(A_log)
    dt_bias = _f64(dt_bias)
    assert b.shape == a.shape and A_log.shape == (H,) and dt_bias.shape == (H,)
    alpha = np.empty_like(a)
    beta = np.empty_like(a)
    g = np.empty_like(a)
    _load().gdn_oracle_gates(_p(a), _p(b), _p(A_log), _p(dt_bias), _p(alpha), _p(beta),
                             _p(g), N, H)
    return alpha, beta, g


def conv_silu(x, w, hist=None):
    """Depthwise causal conv (width W = w.shape[1]) + silu over [B, T, C]
    ("Qwen3.8 27B" card; llm-arch-viz conv1d 10240x1x4, no bias).
    Returns (y [B,T,C], hist_out [B,W-1,C])."""
    x = _f64(x)
    w = _f64(w)
    B, T, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W)
    if hist is not None:
        hist = _f64(hist)
        assert hist.shape == (B, W - 1, C)
    y = np.empty_like(x)
    hist_out = np.empty((B, W - 1, C), dtype=np.float64)
    _load().gdn_oracle_conv_silu(_p(x), _p(w), _p(hist), _p(y), _p(hist_out), B, T, C, W)
    return y, hist_out


def l2norm_heads(y, l2_channels, head_dim, eps=1e-6):
    """Divide each head_dim group of the first l2_channels channels by
    sqrt(sum sq + eps) ("Qwen3.8 27B" card: q and k L2-normalised)."""
    y = _f64(y).copy()
    C = y.shape[-1]
    N = y.size // C
    _load().gdn_oracle_l2norm_heads(_p(y), N, C, l2_channels, head_dim, float(eps))
    return y


def recurrence(q, k, v, alpha, beta, S0=None, q_scale=1.0):
    """Gated delta rule, sequential over tokens.  q, k: [B,T,Hk,dk];
    v: [B,T,Hv,dv]; alpha, beta: [B,T,Hv]; S0: [B,Hv,dv,dk] or None.
    Returns (o [B,T,Hv,dv], S [B,Hv,dv,dk])."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    alpha = _f64(alpha)
    beta = _f64(beta)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T)
    assert alpha.shape == (B, T, Hv) and beta.shape == (B, T, Hv)
    assert Hv % Hk == 0
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (B, Hv, dv, dk)
    o = np.empty((B, T, Hv, dv), dtype=np.float64)
    S = np.empty((B, Hv, dv, dk), dtype=np.float64)
    _load().gdn_oracle_recurrence(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(S0), _p(S),
                                  _p(o), B, T, Hk, Hv, dk, dv, float(q_scale))
    return o, S


def gated_rmsnorm(x, z, w, eps=1e-6):
    """y = x / sqrt(mean(x^2)+eps) * (1+w) * silu(z) per (token, head)
    ("Qwen3.8 27B" card, Gated DeltaNet and Norms bullets).  x, z: [..., H, D];
    w: [D]."""
    x = _f64(x)
    z = _f64(z)
    w = _f64(w)
    D = x.shape[-1]
    H = x.shape[-2]
    N = x.size // (H * D)
    assert z.shape == x.shape and w.shape == (D,)
    y = np.empty_like(x)
    _load().gdn_oracle_gated_rmsnorm(_p(x), _p(z), _p(w), _p(y), N, H, D, float(eps))
    return y


def linear(x, W):
    """y = x W^T, the map of every projection around the mixer ("Qwen/Qwen3.8-27B"
    architecture viewer, module tree: in_proj_qkv, in_proj_z, in_proj_a,
    in_proj_b, out_proj).  x: [..., K]; W: [N, K]; returns [..., N]."""
    x = _f64(x)
    W = _f64(W)
    N, K = W.shape
    assert x.shape[-1] == K
    M = x.size // K if K else 0
    y = np.empty(x.shape[:-1] + (N,), dtype=np.float64)
    if M and N:
        _load().gdn_oracle_linear(_p(x), _p(W), _p(y), M, N, K)
    return y


def mixer(qkv, conv_w, z, a, b, A_log, dt_bias, norm_w, Hk, Hv, d,
          conv_hist=None, S0=None, l2_eps=1e-6, norm_eps=1e-6, q_scale=1.0):
    """The whole mixer path between the projections, in the card's order:
    conv+silu over [q|k|v] channels -> L2 of q and k heads -> gates -> gated
    delta rule -> gated RMSNorm with z.  Channel order [q (Hk*d); k (Hk*d);
    v (Hv*d)].  Returns (y [B,T,Hv*d], S [B,Hv,d,d], conv_hist_out)."""
    B, T, C = qkv.shape
    assert C == 2 * Hk * d + Hv * d
    y, hist_out = conv_silu(qkv, conv_w, conv_hist)
    y = l2norm_heads(y.reshape(B * T, C), 2 * Hk * d, d, l2_eps).reshape(B, T, C)
    q = y[:, :, :Hk * d].reshape(B, T, Hk, d)
    k = y[:, :, Hk * d:2 * Hk * d].reshape(B, T, Hk, d)
    v = y[:, :, 2 * Hk * d:].reshape(B, T, Hv, d)
    alpha, beta, _ = gates(a, b, A_log, dt_bias)
    o, S = recurrence(q, k, v, alpha, beta, S0, q_scale)
    out = gated_rmsnorm(o, _f64(z).reshape(B, T, Hv, d), norm_w, norm_eps)
    return out.reshape(B, T, Hv * d), S, hist_out
