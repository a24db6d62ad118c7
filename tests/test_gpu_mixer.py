"""The whole mixer path and the long prefill, checked against the f64 oracle,
at small sizes and at their full sizes on every (batch, head).

Whole mixer (bf16 in): gdn_mixer_prefill (conv over 10240 channels, width 4,
silu, L2 of q/k -> chunked prefill with the state carried -> gated RMSNorm),
the launch configuration the benchmark times; and the same steps as three
calls (gdn_conv_silu with an f32 output -> gdn_prefill on strided views of it
-> gdn_gated_rmsnorm), where the f32 q/k/v take the sequential f32 kernel.
Long prefill: T=65536 as 16 calls of 4096 with the f32 state handed between
them, against one oracle pass.  The full-size checks compare whole tensors;
the oracle runs one batch row at a time to bound host memory.
Bar: 2e-2 (bf16 inputs), 1e-4 (f32 inputs), max|x-ref|/max|ref| per output
tensor.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import HK, HV, D, make_workload, mixer_inputs, to_f64  # noqa: E402
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

TOL = 2e-2
TOL_F32 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


class RelErr:
    """max|x - ref| / max|ref| of one tensor accumulated over pieces (any
    non-finite x is a failure)."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert x.shape == ref.shape, (x.shape, ref.shape)
        if not np.all(np.isfinite(x)):
            self.num = float("inf")
            return
        self.num = max(self.num, float(np.max(np.abs(x - ref))))
        self.den = max(self.den, float(np.max(np.abs(ref))))

    def value(self):
        return self.num / self.den if self.den > 0 else self.num


def run_mixer_calls(x, B, T, Hk, Hv, d, conv_state=None, S=None):
    """The mixer as three calls: conv (f32 out) -> prefill on views (f32 q/k/v:
    the sequential kernel; bf16 o) -> gated RMSNorm."""
    y = gdn.gdn_conv_silu(dev(x["qkv"]), dev(x["conv_w"]), conv_state, l2_channels=2 * Hk * d,
                          head_dim=d, y_dtype=torch.float32)
    q = y[:, :, :Hk * d].unflatten(2, (Hk, d))
    k = y[:, :, Hk * d:2 * Hk * d].unflatten(2, (Hk, d))
    v = y[:, :, 2 * Hk * d:].unflatten(2, (Hv, d))
    if S is None:
        S = torch.zeros((B, Hv, d, d), dtype=torch.float32, device="cuda")
    o = gdn.gdn_prefill(q, k, v, dev(x["a"]), dev(x["b"]), dev(x["A_log"]), dev(x["dt_bias"]),
                        S, S, algo="auto", o_dtype=torch.bfloat16)
    del y
    out = gdn.gdn_gated_rmsnorm(o, dev(x["z"]).view(B, T, Hv, d), dev(x["norm_w"]))
    torch.cuda.synchronize()
    return out, S


def run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=None, S=None, dtype=None):
    if S is None:
        S = torch.zeros((B, Hv, d, d), dtype=torch.float32, device="cuda")
    qkv, z = dev(x["qkv"]), dev(x["z"])
    if dtype is not None:
        qkv, z = qkv.to(dtype), z.to(dtype)
    y = gdn.gdn_mixer_prefill(qkv, z, dev(x["conv_w"]), dev(x["a"]), dev(x["b"]), dev(x["A_log"]),
                              dev(x["dt_bias"]), dev(x["norm_w"]), Hk, Hv, conv_state=conv_state,
                              state_in=S, state_out=S)
    torch.cuda.synchronize()
    return y, S


def test_mixer_small_all_heads():
    banner("mixer small B=2 T=150 Hk=2 Hv=6: one call and three calls")
    B, T, Hk, Hv, d = 2, 150, 2, 6, 128
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=31)
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                       to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                       x["norm_w"], Hk, Hv, d)
    cs = torch.zeros((B, 3, 2 * Hk * d + Hv * d), dtype=torch.float32, device="cuda")
    out, S = run_mixer_calls(x, B, T, Hk, Hv, d, conv_state=cs)
    assert max_rel_err(host_f64(out).reshape(B, T, Hv * d), y_ref) < TOL
    assert max_rel_err(host_f64(S), S_ref) < TOL
    assert np.array_equal(host_f64(cs), h_ref)
    cs1 = torch.zeros_like(cs)
    y1, S1 = run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=cs1)
    assert max_rel_err(host_f64(y1), y_ref) < TOL
    assert max_rel_err(host_f64(S1), S_ref) < TOL
    assert np.array_equal(host_f64(cs1), h_ref)


@pytest.mark.parametrize("T", [150, 64, 5, 2])
def test_mixer_prefill_one_call_small(T):
    """gdn_mixer_prefill against the oracle (with a carried state and conv
    history), and bitwise repeatable."""
    banner(f"mixer_prefill one call B=2 T={T} Hk=2 Hv=6")
    B, Hk, Hv, d = 2, 2, 6, 128
    C = 2 * Hk * d + Hv * d
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=41 + T)
    rng = np.random.Generator(np.random.PCG64(7 + T))
    S0 = torch.from_numpy(rng.normal(0.0, 0.05, (B, Hv, d, d)).astype(np.float32)).cuda()
    h0 = torch.from_numpy(rng.standard_normal((B, 3, C)).astype(np.float32)).cuda()
    cs1, S1 = h0.clone(), S0.clone()
    y1, S1 = run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=cs1, S=S1)
    cs2, S2 = h0.clone(), S0.clone()
    y2, S2 = run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=cs2, S=S2)
    assert torch.equal(y1, y2) and torch.equal(S1, S2) and torch.equal(cs1, cs2)  # repeatable
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                       to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                       x["norm_w"], Hk, Hv, d, conv_hist=host_f64(h0),
                                       S0=host_f64(S0))
    assert max_rel_err(host_f64(y1), y_ref) < TOL
    assert max_rel_err(host_f64(S1), S_ref) < TOL
    assert np.array_equal(host_f64(cs1), h_ref)


@pytest.mark.parametrize("B,T,dt", [(2, 150, "bf16"), (1, 64, "bf16"), (3, 1, "bf16"),
                                    (2, 70, "f32")])
def test_mixer_prefill_reads_one_projection_buffer(B, T, dt):
    """qkv and z as the two column ranges of one [B, T, C + Hv*128] buffer
    (one in_proj_qkvz product's output): bitwise the result of contiguous
    copies, and within the bar of the oracle (f32 inputs take the sequential
    f32 path, whose conv and norm read the same strided views)."""
    banner(f"mixer_prefill strided qkv/z B={B} T={T} {dt} Hk=2 Hv=6")
    Hk, Hv, d = 2, 6, 128
    C = 2 * Hk * d + Hv * d
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, dt=dt, seed=61 + T)
    buf = torch.cat([dev(x["qkv"]), dev(x["z"])], dim=2)
    qv, zv = buf[..., :C], buf[..., C:]
    rng = np.random.Generator(np.random.PCG64(9 + T))
    S0 = torch.from_numpy(rng.normal(0.0, 0.05, (B, Hv, d, d)).astype(np.float32)).cuda()
    h0 = torch.from_numpy(rng.standard_normal((B, 3, C)).astype(np.float32)).cuda()
    outs = []
    for qkv, z in ((qv, zv), (qv.contiguous(), zv.contiguous())):
        cs, S = h0.clone(), S0.clone()
        y = gdn.gdn_mixer_prefill(qkv, z, dev(x["conv_w"]), dev(x["a"]), dev(x["b"]),
                                  dev(x["A_log"]), dev(x["dt_bias"]), dev(x["norm_w"]), Hk, Hv,
                                  conv_state=cs, state_in=S, state_out=S)
        outs.append((y, S, cs))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                       to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                       x["norm_w"], Hk, Hv, d, conv_hist=host_f64(h0),
                                       S0=host_f64(S0))
    tol = TOL_F32 if dt == "f32" else TOL
    assert max_rel_err(host_f64(outs[0][0]), y_ref) < tol
    assert max_rel_err(host_f64(outs[0][1]), S_ref) < tol
    assert np.array_equal(host_f64(outs[0][2]), h_ref)


def test_mixer_prefill_f32_inputs_and_edge_cases():
    """f32 qkv/z/y (conv, sequential f32 recurrence and norm: the f32 bar
    1e-4), no conv history (NULL: zeros, not written), and T == 0 (state
    passes through)."""
    banner("mixer_prefill f32 B=1 T=100 Hk=2 Hv=6; T=0")
    B, T, Hk, Hv, d = 1, 100, 2, 6, 128
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, dt="f32", seed=53)
    y, S = run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=None)
    assert y.dtype == torch.float32
    y_ref, S_ref, _ = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                   to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                   x["norm_w"], Hk, Hv, d)
    assert max_rel_err(host_f64(y), y_ref) < TOL_F32
    assert max_rel_err(host_f64(S), S_ref) < TOL_F32
    # T == 0: nothing but the state pass-through
    S_in = torch.randn((B, Hv, d, d), dtype=torch.float32, device="cuda")
    S_out = torch.full_like(S_in, float("nan"))
    cs = torch.randn((B, 3, 2 * Hk * d + Hv * d), dtype=torch.float32, device="cuda")
    cs0 = cs.clone()
    e = torch.empty((B, 0, 2 * Hk * d + Hv * d), dtype=torch.bfloat16, device="cuda")
    ez = torch.empty((B, 0, Hv * d), dtype=torch.bfloat16, device="cuda")
    ea = torch.empty((B, 0, Hv), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_mixer_prefill(e, ez, dev(x["conv_w"]), ea, ea, dev(x["A_log"]), dev(x["dt_bias"]),
                          dev(x["norm_w"]), Hk, Hv, conv_state=cs, state_in=S_in,
                          state_out=S_out)
    torch.cuda.synchronize()
    assert torch.equal(S_out, S_in)
    assert torch.equal(cs, cs0)


@pytest.mark.slow
def test_mixer_bf16_b4_t8192_all_heads():
    """The whole-mixer workload at full size (B=4, T=8192, 16/48 heads, 10240
    conv channels), one gdn_mixer_prefill call as the benchmark times it: y,
    the final state and the conv history of every (batch, head) against the
    oracle; a second call gives the same bits."""
    banner("mixer_bf16_b4_t8192 full, every (batch, head)")
    B, T = 4, 8192
    x = make_workload("mixer_bf16_b4_t8192")
    cs = torch.zeros((B, 3, 2 * HK * D + HV * D), dtype=torch.float32, device="cuda")
    y, S = run_mixer_fused(x, B, T, HK, HV, D, conv_state=cs)
    ey, es = RelErr(), RelErr()
    for bb in range(B):
        y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"][bb:bb + 1]), to_f64(x["conv_w"]),
                                           to_f64(x["z"][bb:bb + 1]), to_f64(x["a"][bb:bb + 1]),
                                           to_f64(x["b"][bb:bb + 1]), x["A_log"], x["dt_bias"],
                                           x["norm_w"], HK, HV, D)
        ey.add(host_f64(y[bb:bb + 1]), y_ref)
        es.add(host_f64(S[bb:bb + 1]), S_ref)
        assert np.array_equal(host_f64(cs[bb:bb + 1]), h_ref), bb  # the last 3 inputs, exactly
        del y_ref, S_ref
    print(f"mixer_bf16_b4_t8192: y err {ey.value():.3e}, state err {es.value():.3e}")
    assert ey.value() < TOL and es.value() < TOL
    cs2 = torch.zeros_like(cs)
    y2, S2 = run_mixer_fused(x, B, T, HK, HV, D, conv_state=cs2)
    assert torch.equal(y2, y) and torch.equal(S2, S) and torch.equal(cs2, cs)


def run_long_prefill(x, T, n_calls):
    """T tokens as n_calls sequential gdn_prefill calls with the state handed
    over, as the benchmark times it (one workspace reused)."""
    L = T // n_calls
    qd, kd, vd, ad, bd = (dev(x[n]) for n in ("q", "k", "v", "a", "b"))
    Al, db = dev(x["A_log"]), dev(x["dt_bias"])
    S = torch.zeros((1, HV, D, D), dtype=torch.float32, device="cuda")
    if x.get("state") is not None:
        S.copy_(dev(x["state"]))
    o = torch.empty((1, T, HV, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, L, HK, HV), dtype=torch.uint8,
                     device="cuda")
    for i in range(n_calls):
        sl = slice(i * L, (i + 1) * L)
        gdn.gdn_prefill(qd[:, sl], kd[:, sl], vd[:, sl], ad[:, sl].contiguous(),
                        bd[:, sl].contiguous(), Al, db, S, S, o=o[:, sl], workspace=ws)
    torch.cuda.synchronize()
    return o, S


def oracle_prefill(x):
    al, be, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    S0 = None if x.get("state") is None else to_f64(x["state"])
    return oracle.recurrence(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), al, be, S0)


@pytest.mark.slow
def test_prefill_t65536_as_16_calls_all_heads():
    """Long prefill: 16 sequential 4096-token calls with the f32 state handed
    between them, against one oracle pass over all 65536 tokens, every head."""
    banner("prefill_bf16_b1_t65536_x16 full, every head")
    x = make_workload("prefill_bf16_b1_t65536_x16")
    o, S = run_long_prefill(x, 65536, 16)
    o_ref, S_ref = oracle_prefill(x)
    e_o, e_s = max_rel_err(host_f64(o), o_ref), max_rel_err(host_f64(S), S_ref)
    print(f"prefill_bf16_b1_t65536_x16: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o < TOL and e_s < TOL
