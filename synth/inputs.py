"""Seeded synthetic inputs for the Gated DeltaNet mixer workloads.

Every array is drawn from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order, then rounded to its storage dtype.  bf16 arrays are held as ``uint16``
bit patterns (numpy has no bf16); ``to_f64`` decodes them exactly.  The
rounded values are the inputs of both the GPU path and the oracle.

Distributions (the workload table of the project statement; "N(0, s)" reads
s as the standard deviation):
  q, k   : N(0,1) per element, then each head vector scaled to unit length
           (i.e. uniform direction on the sphere), then rounded.
  v, a, b, z, qkv : N(0,1);  A_log : U(-1,1);  dt_bias : N(0,0.1)
  carried state : N(0,0.05);  conv weights : N(0,0.5) rounded to bf16 and
  stored as f32;  norm weight w : N(0,0.1) (the scale is 1+w).
Dimensions: 16 q/k heads, 48 value heads, width 128, conv 10240 channels of
width 4 ("Qwen3.8 27B" model card, command-line bindings).
"""
import numpy as np

__all__ = ["HK", "HV", "D", "CONV_CH", "CONV_W", "WORKLOADS", "bf16_round", "f32_round",
           "to_f64", "is_bf16", "recurrence_inputs", "decode_inputs", "mixer_inputs",
           "slots_inputs", "decode_multi_inputs", "make_workload", "unit_heads",
           "proj_inputs", "HIDDEN", "correlated_keys_inputs"]

HK, HV, D = 16, 48, 128
HIDDEN = 5120  # model width ("Qwen/Qwen3.8-27B" architecture viewer, header)
CONV_CH = 2 * HK * D + HV * D  # 10240
CONV_W = 4


def f32_round(x):
    """Round to f32 (round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x):
    """Round to bf16 (RNE), returned as uint16 bit patterns.  f64 inputs are
    first rounded to f32 (RNE), then to bf16 (RNE)."""
    f = np.ascontiguousarray(np.asarray(x).astype(np.float32, copy=False))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def is_bf16(a):
    return isinstance(a, np.ndarray) and a.dtype == np.uint16


def to_f64(a):
    """Exact f64 value of an f32 array or of a bf16 bit-pattern array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _round(x, dt):
    if dt == "bf16":
        return bf16_round(x)
    if dt == "f32":
        return f32_round(x)
    raise ValueError(dt)


def unit_heads(x):
    """Scale each vector along the last axis to unit length (the draw of a
    uniformly random direction)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def recurrence_inputs(B, T, Hk=HK, Hv=HV, d=D, qkv_dt="f32", gate_dt="f32", seed=0,
                      state_std=None, A_log_range=(-1.0, 1.0), dt_bias_std=0.1,
                      unit_qk=True):
    """Inputs of one prefill call: q, k [B,T,Hk,d]; v [B,T,Hv,d]; a, b [B,T,Hv];
    A_log, dt_bias [Hv] f32; state [B,Hv,d,d] f32 or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, Hk, d))
    k = rng.standard_normal((B, T, Hk, d))
    if unit_qk:
        q, k = unit_heads(q), unit_heads(k)
    v = rng.standard_normal((B, T, Hv, d))
    a = rng.standard_normal((B, T, Hv))
    b = rng.standard_normal((B, T, Hv))
    A_log = rng.uniform(A_log_range[0], A_log_range[1], Hv)
    dt_bias = rng.normal(0.0, dt_bias_std, Hv)
    state = None if state_std is None else rng.normal(0.0, state_std, (B, Hv, d, d))
    return {
        "q": _round(q, qkv_dt), "k": _round(k, qkv_dt), "v": _round(v, qkv_dt),
        "a": _round(a, gate_dt), "b": _round(b, gate_dt),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "state": None if state is None else f32_round(state),
    }


def correlated_keys_inputs(B, T, Hk=HK, Hv=HV, d=D, spread=0.1, b_mean=6.0,
                           A_log_range=(-6.0, -4.0), qkv_dt="bf16", gate_dt="f32", seed=9,
                           state_std=0.05):
    """Prefill inputs whose keys are nearly parallel within each (batch, q/k
    head): k_t = unit(u + spread * n_t / sqrt(d)) with one random unit u per
    (batch, q/k head) and n_t ~ N(0, I); b ~ N(b_mean, 0.5) (write rates near
    1) and A_log ~ U(A_log_range) (slow decay).  With the defaults, pairs of
    keys have k.k ~ 0.99.  q: unit random; v, a: N(0,1); dt_bias N(0, 0.1);
    state N(0, state_std) or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = unit_heads(rng.standard_normal((B, 1, Hk, d)))
    k = unit_heads(u + spread * rng.standard_normal((B, T, Hk, d)) / np.sqrt(d))
    q = unit_heads(rng.standard_normal((B, T, Hk, d)))
    v = rng.standard_normal((B, T, Hv, d))
    a = rng.standard_normal((B, T, Hv))
    b = rng.normal(b_mean, 0.5, (B, T, Hv))
    A_log = rng.uniform(A_log_range[0], A_log_range[1], Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    state = None if state_std is None else rng.normal(0.0, state_std, (B, Hv, d, d))
    return {
        "q": _round(q, qkv_dt), "k": _round(k, qkv_dt), "v": _round(v, qkv_dt),
        "a": _round(a, gate_dt), "b": _round(b, gate_dt),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "state": None if state is None else f32_round(state),
    }


def slots_inputs(lengths, Hk=HK, Hv=HV, d=D, qkv_dt="bf16", gate_dt="f32", seed=5,
                 state_std=0.05):
    """Inputs of one ragged prefill of fixed rows: row r brings lengths[r] new
    tokens.  The tokens are packed row after row: q, k [N,Hk,d]; v [N,Hv,d];
    a, b [N,Hv]; cu_seqlens [R+1] int32 (row r is tokens cu[r]..cu[r+1]);
    A_log, dt_bias [Hv] f32; state [R,Hv,d,d] f32 (each row's carried state)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    R, N = len(lengths), int(lengths.sum())
    cu = np.zeros(R + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q = unit_heads(rng.standard_normal((N, Hk, d)))
    k = unit_heads(rng.standard_normal((N, Hk, d)))
    v = rng.standard_normal((N, Hv, d))
    a = rng.standard_normal((N, Hv))
    b = rng.standard_normal((N, Hv))
    A_log = rng.uniform(-1.0, 1.0, Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    state = rng.standard_normal((R, Hv, d, d), dtype=np.float32) * np.float32(state_std)
    return {
        "q": _round(q, qkv_dt), "k": _round(k, qkv_dt), "v": _round(v, qkv_dt),
        "a": _round(a, gate_dt), "b": _round(b, gate_dt),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "state": state.astype(np.float32), "cu_seqlens": cu, "max_len": int(lengths.max(initial=0)),
    }


def decode_multi_inputs(R, K, Hk=HK, Hv=HV, d=D, qkv_dt="bf16", gate_dt="bf16", seed=6,
                        state_std=0.05, max_len=8192):
    """Inputs of one multi-token decode_rows call: K draft tokens per fixed row.
    q, k [R,K,Hk,d]; v [R,K,Hv,d]; a, b [R,K,Hv]; A_log, dt_bias [Hv];
    state [R,Hv,d,d] f32; lengths [R] int32 ~ U{1..max_len}."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = unit_heads(rng.standard_normal((R, K, Hk, d)))
    k = unit_heads(rng.standard_normal((R, K, Hk, d)))
    v = rng.standard_normal((R, K, Hv, d))
    a = rng.standard_normal((R, K, Hv))
    b = rng.standard_normal((R, K, Hv))
    A_log = rng.uniform(-1.0, 1.0, Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    lengths = rng.integers(1, max_len + 1, R).astype(np.int32)
    state = rng.standard_normal((R, Hv, d, d), dtype=np.float32) * np.float32(state_std)
    return {
        "q": _round(q, qkv_dt), "k": _round(k, qkv_dt), "v": _round(v, qkv_dt),
        "a": _round(a, gate_dt), "b": _round(b, gate_dt),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "state": state.astype(np.float32), "lengths": lengths,
    }


def decode_inputs(R, Hk=HK, Hv=HV, d=D, qkv_dt="bf16", gate_dt="bf16", seed=1,
                  state_std=0.05, max_len=8192):
    """Inputs of one decode_rows call: q, k [R,Hk,d]; v [R,Hv,d]; a, b [R,Hv];
    A_log, dt_bias [Hv]; state [R,Hv,d,d] f32; lengths [R] int32 ~ U{1..max_len}."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = unit_heads(rng.standard_normal((R, Hk, d)))
    k = unit_heads(rng.standard_normal((R, Hk, d)))
    v = rng.standard_normal((R, Hv, d))
    a = rng.standard_normal((R, Hv))
    b = rng.standard_normal((R, Hv))
    A_log = rng.uniform(-1.0, 1.0, Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    lengths = rng.integers(1, max_len + 1, R).astype(np.int32)
    state = rng.standard_normal((R, Hv, d, d), dtype=np.float32) * np.float32(state_std)
    return {
        "q": _round(q, qkv_dt), "k": _round(k, qkv_dt), "v": _round(v, qkv_dt),
        "a": _round(a, gate_dt), "b": _round(b, gate_dt),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "state": state.astype(np.float32), "lengths": lengths,
    }


def mixer_inputs(B, T, Hk=HK, Hv=HV, d=D, dt="bf16", seed=3, conv_w_std=0.5,
                 norm_w_std=0.1):
    """Inputs of the whole mixer: qkv [B,T,2*Hk*d+Hv*d]; conv_w [C,4] f32
    (bf16-rounded values); z [B,T,Hv*d]; a, b [B,T,Hv]; A_log, dt_bias [Hv];
    norm_w [d] f32.  Big arrays are drawn in f32 to bound host memory."""
    rng = np.random.Generator(np.random.PCG64(seed))
    C = 2 * Hk * d + Hv * d
    qkv = rng.standard_normal((B, T, C), dtype=np.float32)
    conv_w = rng.normal(0.0, conv_w_std, (C, CONV_W))
    z = rng.standard_normal((B, T, Hv * d), dtype=np.float32)
    a = rng.standard_normal((B, T, Hv))
    b = rng.standard_normal((B, T, Hv))
    A_log = rng.uniform(-1.0, 1.0, Hv)
    dt_bias = rng.normal(0.0, 0.1, Hv)
    norm_w = rng.normal(0.0, norm_w_std, d)
    return {
        "qkv": _round(qkv, dt), "z": _round(z, dt), "a": _round(a, dt), "b": _round(b, dt),
        "conv_w": to_f64(bf16_round(conv_w)).astype(np.float32),
        "A_log": f32_round(A_log), "dt_bias": f32_round(dt_bias),
        "norm_w": f32_round(norm_w),
    }


def proj_inputs(M, K=HIDDEN, outs=(("W_qkv", CONV_CH), ("W_z", HV * D)), gate_H=HV, seed=7,
                x_name="x"):
    """Inputs of the projections around the mixer: activations x [M, K] ~ N(0,1)
    in bf16; bf16 weights [N, K] ~ N(0, 1/K) (unit-variance outputs), one per
    (name, N) in ``outs``; f32 gate weights W_a, W_b [gate_H, K] ~ N(0, 1/K)
    when gate_H > 0.  Drawn in f32 to bound host memory."""
    rng = np.random.Generator(np.random.PCG64(seed))
    res = {x_name: bf16_round(rng.standard_normal((M, K), dtype=np.float32))}
    s = np.float32(1.0 / np.sqrt(K))
    for name, N in outs:
        res[name] = bf16_round(rng.standard_normal((N, K), dtype=np.float32) * s)
    if gate_H:
        res["W_a"] = rng.standard_normal((gate_H, K), dtype=np.float32) * s
        res["W_b"] = rng.standard_normal((gate_H, K), dtype=np.float32) * s
    return res


# The five workloads, by name.  Sizes follow the model's layer; the seeds are
# fixed so every run (tests, bench, oracle) sees identical inputs.
WORKLOADS = {
    "recurrence_f32_b1_t64": dict(kind="prefill", B=1, T=64, qkv_dt="f32", gate_dt="f32",
                                  state_std=None, seed=1000),
    "decode_rows_r64": dict(kind="decode", R=64, qkv_dt="bf16", gate_dt="bf16", seed=1001),
    "prefill_bf16_b1_t4096": dict(kind="prefill", B=1, T=4096, qkv_dt="bf16", gate_dt="f32",
                                  state_std=0.05, seed=1002),
    "mixer_bf16_b4_t8192": dict(kind="mixer", B=4, T=8192, dt="bf16", seed=1003),
    "prefill_bf16_b1_t65536_x16": dict(kind="prefill", B=1, T=65536, qkv_dt="bf16",
                                       gate_dt="f32", state_std=None, seed=1004,
                                       calls=16),
    # Verifying a 4-token draft on 64 fixed rows (the decode workload's shape).
    "decode_rows_r64_k4": dict(kind="decode_multi", R=64, K=4, qkv_dt="bf16", gate_dt="bf16",
                               seed=1006),
    # A server's ragged prefill: 16 fixed rows, new-token counts ~ U{1..1024}
    # drawn from the seed's first integers, states ~ N(0, 0.05).
    "prefill_slots_bf16_r16": dict(kind="slots", R=16, max_new=1024, qkv_dt="bf16",
                                   gate_dt="f32", seed=1005),
}


def make_workload(name, **overrides):
    """Inputs of a named workload; keyword overrides (e.g. a smaller T) allowed."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    cfg.pop("calls", None)
    if kind == "prefill":
        return recurrence_inputs(**cfg)
    if kind == "decode":
        return decode_inputs(**cfg)
    if kind == "mixer":
        return mixer_inputs(**cfg)
    if kind == "decode_multi":
        return decode_multi_inputs(**cfg)
    if kind == "slots":
        rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
        lengths = rng.integers(1, cfg.pop("max_new") + 1, cfg.pop("R"))
        return slots_inputs(lengths, **cfg)
    raise ValueError(kind)
