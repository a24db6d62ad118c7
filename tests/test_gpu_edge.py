"""Edge cases of the hot path on the GPU, each against the f64 oracle:

* gates at +-inf through every entry point (a = +inf or A_log = +inf: alpha = 0,
  the state restarts; a = -inf or A_log = -inf: alpha = 1; b = +inf: beta = 1;
  b = -inf: beta = 0, the state only decays) -- "Qwen3.8 27B" model card,
  Gated DeltaNet bullet (the gate definitions);
* one q/k head per value head (Hv == Hk);
* nearly parallel keys, where I + A of the chunk form has a condition number
  near 80 and W = T diag(b gamma) K is a difference of nearly equal rows;
* slow decay (A_log ~ U(-6, -4), alpha ~ 0.99) over 4096 tokens in one call
  and over 65536 tokens in 16 calls with the state handed over;
* guard bands: 256 bytes before and after every output buffer (and the
  workspace) keep their bit pattern.

Bar: 2e-2 for bf16 inputs, 1e-4 for f32 inputs (max|x-ref|/max|ref| per output
tensor); outputs must be finite.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import (correlated_keys_inputs, decode_inputs, decode_multi_inputs,  # noqa: E402
                   mixer_inputs, recurrence_inputs, slots_inputs, to_f64)
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

TOL = {"bf16": 2e-2, "f32": 1e-4}
BF16_INF, BF16_NINF = 0x7F80, 0xFF80


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _ref(x, S0=None, q_scale=1.0):
    al, be, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    return oracle.recurrence(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), al, be, S0,
                             q_scale=q_scale)


def _set(arr, idx, val):
    """Write +-inf into a gate array held as f32 or as bf16 bit patterns."""
    if arr.dtype == np.uint16:
        arr[idx] = BF16_INF if val > 0 else BF16_NINF
    else:
        arr[idx] = val


def with_inf_gates(x, tok_axis=1):
    """A copy of prefill-shaped inputs (gates [B, T, Hv], Hv >= 6, B >= 2,
    T >= 130) with infinite gates placed on both sides of the first chunk
    boundary (token 64):
      a = +inf  at (0, 10, h0) and (0, 60..69, h1)   -> alpha = 0
      a = -inf  at (1, 5, h2) and (1, 64..129, h2)   -> alpha = 1
      b = +inf  at (0, 20, h3); b = -inf at (1, 100, h3)
      b = -inf  on tokens 0..63 of head 5            -> beta = 0
      A_log = +inf on head 4 (alpha = 0 at every token), -inf on head 5."""
    y = {n: (v.copy() if isinstance(v, np.ndarray) else v) for n, v in x.items()}
    a, b = y["a"], y["b"]
    _set(a, (0, 10, 0), np.inf)
    _set(a, (0, slice(60, 70), 1), np.inf)
    _set(a, (1, 5, 2), -np.inf)
    _set(a, (1, slice(64, 130), 2), -np.inf)
    _set(b, (0, 20, 3), np.inf)
    _set(b, (1, 100, 3), -np.inf)
    _set(b, (slice(None), slice(0, 64), 5), -np.inf)
    y["A_log"] = y["A_log"].copy()
    y["A_log"][4] = np.inf
    y["A_log"][5] = -np.inf
    return y


def _finite(t):
    return bool(torch.isfinite(t.float()).all())


# ------------------------------------------------------------------ +-inf gates

@pytest.mark.parametrize("qkv_dt,gate_dt", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32"),
                                            ("f32", "bf16")])
def test_inf_gates_prefill(qkv_dt, gate_dt):
    """bf16 q/k/v run the chunked algorithm, f32 q/k/v the sequential one."""
    banner(f"inf gates prefill qkv={qkv_dt} gates={gate_dt}")
    x = with_inf_gates(recurrence_inputs(2, 150, Hk=2, Hv=6, qkv_dt=qkv_dt, gate_dt=gate_dt,
                                         seed=71, state_std=0.05))
    si = dev(x["state"])
    so = torch.empty_like(si)
    o = gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), si, so)
    torch.cuda.synchronize()
    assert _finite(o) and _finite(so)
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    assert np.all(np.isfinite(o_ref)) and np.all(np.isfinite(S_ref))
    assert max_rel_err(host_f64(o), o_ref) < TOL[qkv_dt]
    assert max_rel_err(host_f64(so), S_ref) < TOL[qkv_dt]
    # head 4 restarts at every token (alpha = 0): its final state is
    # beta v k^T of the last token alone
    assert max_rel_err(host_f64(so)[:, 4], S_ref[:, 4]) < TOL[qkv_dt]


@pytest.mark.parametrize("qkv_dt", ["bf16", "f32"])
def test_inf_gates_prefill_slots(qkv_dt):
    banner(f"inf gates prefill_slots {qkv_dt}")
    lengths = [150, 140]
    x = slots_inputs(lengths, Hk=2, Hv=6, qkv_dt=qkv_dt, gate_dt="f32", seed=72)
    cu = x["cu_seqlens"]
    # the same infinite gates, placed per row on the packed axis
    g = {"a": np.zeros((2, 150, 6), np.float32), "b": np.zeros((2, 150, 6), np.float32)}
    for r, L in enumerate(lengths):
        g["a"][r, :L] = x["a"][cu[r]:cu[r + 1]]
        g["b"][r, :L] = x["b"][cu[r]:cu[r + 1]]
    g = with_inf_gates({"a": g["a"], "b": g["b"], "A_log": x["A_log"]})
    for r, L in enumerate(lengths):
        x["a"][cu[r]:cu[r + 1]] = g["a"][r, :L]
        x["b"][cu[r]:cu[r + 1]] = g["b"][r, :L]
    x["A_log"] = g["A_log"]
    st = dev(x["state"])
    o = gdn.gdn_prefill_slots(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                              dev(x["A_log"]), dev(x["dt_bias"]), dev(cu), st, x["max_len"])
    torch.cuda.synchronize()
    assert _finite(o) and _finite(st)
    for r in range(len(lengths)):
        c0, c1 = int(cu[r]), int(cu[r + 1])
        row = {n: x[n][c0:c1][None] for n in ("q", "k", "v", "a", "b")}
        row.update(A_log=x["A_log"], dt_bias=x["dt_bias"])
        o_ref, S_ref = _ref(row, to_f64(x["state"][r:r + 1]))
        assert max_rel_err(host_f64(o[c0:c1]), o_ref[0]) < TOL[qkv_dt], r
        assert max_rel_err(host_f64(st[r:r + 1]), S_ref) < TOL[qkv_dt], r


@pytest.mark.parametrize("qkv_dt,gate_dt", [("bf16", "bf16"), ("f32", "f32")])
def test_inf_gates_decode_rows(qkv_dt, gate_dt):
    banner(f"inf gates decode_rows {qkv_dt}/{gate_dt}")
    x = decode_inputs(6, Hk=2, Hv=6, qkv_dt=qkv_dt, gate_dt=gate_dt, seed=73)
    a, b = x["a"], x["b"]
    _set(a, (0, 0), np.inf)
    _set(a, (1, 2), -np.inf)
    _set(b, (2, 3), np.inf)
    _set(b, (3, 1), -np.inf)
    x["A_log"] = x["A_log"].copy()
    x["A_log"][4] = np.inf
    x["A_log"][5] = -np.inf
    st = dev(x["state"])
    o = gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(a), dev(b),
                            dev(x["A_log"]), dev(x["dt_bias"]), st)
    torch.cuda.synchronize()
    assert _finite(o) and _finite(st)
    al, be, _ = oracle.gates(to_f64(a)[:, None], to_f64(b)[:, None], x["A_log"], x["dt_bias"])
    o_ref, S_ref = oracle.recurrence(to_f64(x["q"])[:, None], to_f64(x["k"])[:, None],
                                     to_f64(x["v"])[:, None], al, be, to_f64(x["state"]))
    assert max_rel_err(host_f64(o), o_ref[:, 0]) < TOL[qkv_dt]
    assert max_rel_err(host_f64(st), S_ref) < 1e-5


def test_inf_gates_decode_rows_multi():
    banner("inf gates decode_rows_multi K=4")
    x = decode_multi_inputs(3, 4, Hk=2, Hv=6, seed=74)
    a, b = x["a"], x["b"]
    _set(a, (0, 1, 0), np.inf)
    _set(a, (1, slice(0, 3), 2), -np.inf)
    _set(b, (2, 2, 3), np.inf)
    _set(b, (0, slice(None), 1), -np.inf)
    st = dev(x["state"])
    o = gdn.gdn_decode_rows_multi(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(a), dev(b),
                                  dev(x["A_log"]), dev(x["dt_bias"]), st)
    torch.cuda.synchronize()
    assert _finite(o) and _finite(st)
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    assert max_rel_err(host_f64(o), o_ref) < TOL["bf16"]
    assert max_rel_err(host_f64(st), S_ref) < 1e-5


def test_inf_gates_mixer_prefill():
    banner("inf gates mixer_prefill bf16 B=2 T=150")
    B, T, Hk, Hv, d = 2, 150, 2, 6, 128
    x = with_inf_gates(mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=75))
    S = torch.zeros((B, Hv, d, d), dtype=torch.float32, device="cuda")
    y = gdn.gdn_mixer_prefill(dev(x["qkv"]), dev(x["z"]), dev(x["conv_w"]), dev(x["a"]),
                              dev(x["b"]), dev(x["A_log"]), dev(x["dt_bias"]), dev(x["norm_w"]),
                              Hk, Hv, state_in=S, state_out=S)
    torch.cuda.synchronize()
    assert _finite(y) and _finite(S)
    y_ref, S_ref, _ = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                   to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                   x["norm_w"], Hk, Hv, d)
    assert max_rel_err(host_f64(y), y_ref) < TOL["bf16"]
    assert max_rel_err(host_f64(S), S_ref) < TOL["bf16"]


# ------------------------------------------------------------------ Hv == Hk

@pytest.mark.parametrize("B,H,T,qkv_dt", [(2, 4, 150, "bf16"), (1, 16, 130, "bf16"),
                                          (2, 4, 70, "f32")])
def test_one_qk_head_per_value_head_prefill(B, H, T, qkv_dt):
    """Hv == Hk; B*Hk = 16 takes the XCD-grouped workgroup order with groups
    of one value head."""
    banner(f"Hv == Hk = {H} prefill B={B} T={T} {qkv_dt}")
    x = recurrence_inputs(B, T, Hk=H, Hv=H, qkv_dt=qkv_dt, gate_dt="f32", seed=80 + H,
                          state_std=0.05)
    si = dev(x["state"])
    so = torch.empty_like(si)
    o = gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), si, so)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    assert max_rel_err(host_f64(o), o_ref) < TOL[qkv_dt]
    assert max_rel_err(host_f64(so), S_ref) < TOL[qkv_dt]


def test_one_qk_head_per_value_head_decode_and_mixer():
    banner("Hv == Hk = 4 decode_rows, decode_rows_multi, prefill_slots, mixer_prefill")
    H, d = 4, 128
    x = decode_inputs(5, Hk=H, Hv=H, seed=84)
    st = dev(x["state"])
    o = gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                            dev(x["A_log"]), dev(x["dt_bias"]), st)
    torch.cuda.synchronize()
    al, be, _ = oracle.gates(to_f64(x["a"])[:, None], to_f64(x["b"])[:, None], x["A_log"],
                             x["dt_bias"])
    o_ref, S_ref = oracle.recurrence(to_f64(x["q"])[:, None], to_f64(x["k"])[:, None],
                                     to_f64(x["v"])[:, None], al, be, to_f64(x["state"]))
    assert max_rel_err(host_f64(o), o_ref[:, 0]) < TOL["bf16"]
    assert max_rel_err(host_f64(st), S_ref) < 1e-5

    xm = decode_multi_inputs(3, 3, Hk=H, Hv=H, seed=85)
    st = dev(xm["state"])
    o = gdn.gdn_decode_rows_multi(dev(xm["q"]), dev(xm["k"]), dev(xm["v"]), dev(xm["a"]),
                                  dev(xm["b"]), dev(xm["A_log"]), dev(xm["dt_bias"]), st)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(xm, to_f64(xm["state"]))
    assert max_rel_err(host_f64(o), o_ref) < TOL["bf16"]
    assert max_rel_err(host_f64(st), S_ref) < 1e-5

    xs = slots_inputs([70, 0, 130], Hk=H, Hv=H, seed=86)
    st = dev(xs["state"])
    o = gdn.gdn_prefill_slots(dev(xs["q"]), dev(xs["k"]), dev(xs["v"]), dev(xs["a"]),
                              dev(xs["b"]), dev(xs["A_log"]), dev(xs["dt_bias"]),
                              dev(xs["cu_seqlens"]), st, xs["max_len"])
    torch.cuda.synchronize()
    cu = xs["cu_seqlens"]
    for r in (0, 2):
        c0, c1 = int(cu[r]), int(cu[r + 1])
        row = {n: xs[n][c0:c1][None] for n in ("q", "k", "v", "a", "b")}
        row.update(A_log=xs["A_log"], dt_bias=xs["dt_bias"])
        o_ref, S_ref = _ref(row, to_f64(xs["state"][r:r + 1]))
        assert max_rel_err(host_f64(o[c0:c1]), o_ref[0]) < TOL["bf16"], r
        assert max_rel_err(host_f64(st[r:r + 1]), S_ref) < TOL["bf16"], r
    assert torch.equal(st[1], dev(xs["state"][1]))

    B, T = 2, 100
    xx = mixer_inputs(B, T, Hk=H, Hv=H, d=d, seed=87)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    y = gdn.gdn_mixer_prefill(dev(xx["qkv"]), dev(xx["z"]), dev(xx["conv_w"]), dev(xx["a"]),
                              dev(xx["b"]), dev(xx["A_log"]), dev(xx["dt_bias"]),
                              dev(xx["norm_w"]), H, H, state_in=S, state_out=S)
    torch.cuda.synchronize()
    y_ref, S_ref, _ = oracle.mixer(to_f64(xx["qkv"]), to_f64(xx["conv_w"]), to_f64(xx["z"]),
                                   to_f64(xx["a"]), to_f64(xx["b"]), xx["A_log"], xx["dt_bias"],
                                   xx["norm_w"], H, H, d)
    assert max_rel_err(host_f64(y), y_ref) < TOL["bf16"]
    assert max_rel_err(host_f64(S), S_ref) < TOL["bf16"]


# ------------------------------------------------------------------ nearly parallel keys

def chunk_condition(x, b=0, h=0, chunk=64):
    """cond_2(I + A) of the first chunk of (batch b, value head h), in f64 from
    the inputs: A_tj = beta_t e^{G_t - G_j} (k_t . k_j) for j < t."""
    Hv, Hk = x["v"].shape[2], x["k"].shape[2]
    k = to_f64(x["k"][b, :chunk, h // (Hv // Hk)])
    al, be, g = oracle.gates(to_f64(x["a"][b:b + 1, :chunk]), to_f64(x["b"][b:b + 1, :chunk]),
                             x["A_log"], x["dt_bias"])
    G = np.cumsum(g[0, :, h])
    A = np.tril(be[0, :, h][:, None] * np.exp(G[:, None] - G[None, :]) * (k @ k.T), -1)
    return float(np.linalg.cond(np.eye(chunk) + A))


@pytest.mark.parametrize("B,Hk,Hv,T", [(2, 2, 6, 256), (1, 16, 48, 1024)])
def test_nearly_parallel_keys(B, Hk, Hv, T):
    banner(f"nearly parallel keys B={B} Hk={Hk} Hv={Hv} T={T}")
    x = correlated_keys_inputs(B, T, Hk=Hk, Hv=Hv, seed=90 + T)
    conds = [chunk_condition(x, 0, h) for h in range(min(Hv, 6))]
    print("cond(I + A), first chunk:", [round(c, 1) for c in conds])
    assert 40.0 < max(conds) < 400.0  # the conditioning this test is about
    si = dev(x["state"])
    so = torch.empty_like(si)
    o = gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), si, so)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    e_o, e_s = max_rel_err(host_f64(o), o_ref), max_rel_err(host_f64(so), S_ref)
    print(f"nearly parallel keys: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]


# ------------------------------------------------------------------ slow decay, long

def test_slow_decay_t4096_one_call():
    """A_log ~ U(-6, -4): alpha ~ 0.99, so the carried state and every chunk's
    rounding persist over many chunks (64 chunks, model-size heads)."""
    banner("slow decay B=1 T=4096, 16/48 heads")
    x = recurrence_inputs(1, 4096, qkv_dt="bf16", gate_dt="f32", seed=1102, state_std=0.05,
                          A_log_range=(-6.0, -4.0))
    si = dev(x["state"])
    so = torch.empty_like(si)
    o = gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), si, so)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    e_o, e_s = max_rel_err(host_f64(o), o_ref), max_rel_err(host_f64(so), S_ref)
    print(f"slow decay T=4096: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]


@pytest.mark.slow
def test_slow_decay_t65536_as_16_calls():
    """65536 tokens as 16 calls of 4096 with the state handed over, slow decay
    and a carried initial state, every head against one oracle pass."""
    banner("slow decay B=1 T=65536 as 16 x 4096, 16/48 heads")
    T, n_calls = 65536, 16
    L = T // n_calls
    x = recurrence_inputs(1, T, qkv_dt="bf16", gate_dt="f32", seed=1104, state_std=0.05,
                          A_log_range=(-6.0, -4.0))
    qd, kd, vd, ad, bd = (dev(x[n]) for n in ("q", "k", "v", "a", "b"))
    Al, db = dev(x["A_log"]), dev(x["dt_bias"])
    S = dev(x["state"])
    o = torch.empty((1, T, 48, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, L, 16, 48), dtype=torch.uint8,
                     device="cuda")
    for i in range(n_calls):
        sl = slice(i * L, (i + 1) * L)
        gdn.gdn_prefill(qd[:, sl], kd[:, sl], vd[:, sl], ad[:, sl].contiguous(),
                        bd[:, sl].contiguous(), Al, db, S, S, o=o[:, sl], workspace=ws)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(x, to_f64(x["state"]))
    e_o, e_s = max_rel_err(host_f64(o), o_ref), max_rel_err(host_f64(S), S_ref)
    print(f"slow decay T=65536 x16: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]


# ------------------------------------------------------------------ guard bands

GUARD = 256  # bytes before and after each buffer
_SENT = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float32: (torch.int32, 0x7FA5A5A5),
         torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """A device buffer with GUARD bytes of a fixed bit pattern on each side;
    .t is the [shape] tensor in between (256-byte aligned, contiguous)."""

    def __init__(self, shape, dtype, init=None):
        esz = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD // esz
        self.n = int(np.prod(shape)) if len(shape) else 1
        self.buf = torch.empty(self.n + 2 * self.g, dtype=dtype, device="cuda")
        it, val = _SENT[dtype]
        self.raw = self.buf.view(it)
        self.val = val if it is not torch.int16 else val
        self.raw.fill_(val)
        self.t = self.buf[self.g:self.g + self.n].view(shape)
        if init is not None:
            self.t.copy_(init)

    def intact(self):
        lo = self.raw[:self.g]
        hi = self.raw[self.g + self.n:]
        return bool((lo == self.val).all()) and bool((hi == self.val).all())


def test_guard_bands_prefill_chunked_and_sequential():
    banner("guard bands: gdn_prefill chunked (bf16) and sequential (f32)")
    B, T, Hk, Hv = 2, 150, 2, 6
    for qkv_dt in ("bf16", "f32"):
        x = recurrence_inputs(B, T, Hk=Hk, Hv=Hv, qkv_dt=qkv_dt, gate_dt="f32", seed=95,
                              state_std=0.05)
        odt = torch.bfloat16 if qkv_dt == "bf16" else torch.float32
        o = Guarded((B, T, Hv, 128), odt)
        st = Guarded((B, Hv, 128, 128), torch.float32, dev(x["state"]))
        need = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv,
                                               qkv_dtype=odt)
        ws = Guarded((max(need, 1),), torch.uint8)
        gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), st.t, st.t, o=o.t,
                        workspace=ws.t if need else None)
        torch.cuda.synchronize()
        assert o.intact() and st.intact() and ws.intact(), qkv_dt
        o_ref, S_ref = _ref(x, to_f64(x["state"]))
        assert max_rel_err(host_f64(o.t), o_ref) < TOL[qkv_dt]
        assert max_rel_err(host_f64(st.t), S_ref) < TOL[qkv_dt]


def test_guard_bands_decode_conv_norm_slots_mixer():
    banner("guard bands: decode_rows, decode_rows_multi, conv, norm, slots, mixer")
    Hk, Hv, d = 2, 6, 128
    # decode_rows
    x = decode_inputs(3, Hk=Hk, Hv=Hv, seed=96)
    o = Guarded((3, Hv, d), torch.bfloat16)
    st = Guarded((3, Hv, d, d), torch.float32, dev(x["state"]))
    gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), st.t, o=o.t)
    torch.cuda.synchronize()
    assert o.intact() and st.intact()
    # decode_rows_multi with snapshots
    xm = decode_multi_inputs(2, 3, Hk=Hk, Hv=Hv, seed=97)
    o = Guarded((2, 3, Hv, d), torch.bfloat16)
    st = Guarded((2, Hv, d, d), torch.float32, dev(xm["state"]))
    sn = Guarded((2, 3, Hv, d, d), torch.float32)
    gdn.gdn_decode_rows_multi(dev(xm["q"]), dev(xm["k"]), dev(xm["v"]), dev(xm["a"]),
                              dev(xm["b"]), dev(xm["A_log"]), dev(xm["dt_bias"]), st.t, sn.t,
                              o=o.t)
    torch.cuda.synchronize()
    assert o.intact() and st.intact() and sn.intact()
    # conv + silu + L2 with history, and the gated RMSNorm
    B, T = 2, 37
    C = 2 * Hk * d + Hv * d
    xx = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=98)
    y = Guarded((B, T, C), torch.bfloat16)
    cs = Guarded((B, 3, C), torch.float32, torch.randn(B, 3, C, device="cuda"))
    gdn.gdn_conv_silu(dev(xx["qkv"]), dev(xx["conv_w"]), cs.t, l2_channels=2 * Hk * d, y=y.t)
    torch.cuda.synchronize()
    assert y.intact() and cs.intact()
    yn = Guarded((B, T, Hv, d), torch.bfloat16)
    gdn.gdn_gated_rmsnorm(y.t[:, :, 2 * Hk * d:].contiguous().view(B, T, Hv, d),
                          dev(xx["z"]).view(B, T, Hv, d), dev(xx["norm_w"]), y=yn.t)
    torch.cuda.synchronize()
    assert yn.intact()
    # prefill_slots
    xs = slots_inputs([65, 0, 3], Hk=Hk, Hv=Hv, seed=99)
    N = int(xs["cu_seqlens"][-1])
    o = Guarded((N, Hv, d), torch.bfloat16)
    st = Guarded((3, Hv, d, d), torch.float32, dev(xs["state"]))
    need = gdn.gdn_prefill_slots_workspace_bytes(3, xs["max_len"], Hk, Hv)
    ws = Guarded((need,), torch.uint8)
    gdn.gdn_prefill_slots(dev(xs["q"]), dev(xs["k"]), dev(xs["v"]), dev(xs["a"]), dev(xs["b"]),
                          dev(xs["A_log"]), dev(xs["dt_bias"]), dev(xs["cu_seqlens"]), st.t,
                          xs["max_len"], o=o.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert o.intact() and st.intact() and ws.intact()
    # the whole mixer
    yb = Guarded((B, T, Hv * d), torch.bfloat16)
    cs = Guarded((B, 3, C), torch.float32, torch.zeros(B, 3, C, device="cuda"))
    S = Guarded((B, Hv, d, d), torch.float32, torch.zeros(B, Hv, d, d, device="cuda"))
    need = gdn.gdn_mixer_prefill_workspace_bytes(B, T, Hk, Hv)
    ws = Guarded((need,), torch.uint8)
    gdn.gdn_mixer_prefill(dev(xx["qkv"]), dev(xx["z"]), dev(xx["conv_w"]), dev(xx["a"]),
                          dev(xx["b"]), dev(xx["A_log"]), dev(xx["dt_bias"]), dev(xx["norm_w"]),
                          Hk, Hv, conv_state=cs.t, state_in=S.t, state_out=S.t, y=yb.t,
                          workspace=ws.t)
    torch.cuda.synchronize()
    assert yb.intact() and cs.intact() and S.intact() and ws.intact()
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(xx["qkv"]), to_f64(xx["conv_w"]), to_f64(xx["z"]),
                                       to_f64(xx["a"]), to_f64(xx["b"]), xx["A_log"],
                                       xx["dt_bias"], xx["norm_w"], Hk, Hv, d)
    assert max_rel_err(host_f64(yb.t), y_ref) < TOL["bf16"]
    assert max_rel_err(host_f64(S.t), S_ref) < TOL["bf16"]
    assert np.array_equal(host_f64(cs.t), h_ref)
