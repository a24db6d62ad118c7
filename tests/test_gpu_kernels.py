"""GPU parity of the HBM-bound kernels and the sequential recurrence against
the f64 oracle, through the C ABI (via the ctypes binding).

Bar (max|x - ref| / max|ref| per output tensor): 1e-4 for f32 inputs, 2e-2 for
bf16 inputs; the f32 state of decode_rows is also held to 1e-5.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import decode_inputs, make_workload, mixer_inputs, recurrence_inputs, to_f64  # noqa: E402
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


# ------------------------------------------------------------------ conv + silu + L2

@pytest.mark.parametrize("dt,ydt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("T,with_hist", [(150, True), (150, False), (1, True), (2, True), (64, True)])
def test_conv_silu_parity(dt, ydt, T, with_hist):
    banner(f"conv_silu dt={dt} y={ydt} T={T} hist={with_hist}")
    Hk, Hv, d, B = 2, 6, 128, 2
    C = 2 * Hk * d + Hv * d
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, dt=dt, seed=T)
    rng = np.random.default_rng(T)
    hist = rng.normal(size=(B, 3, C)).astype(np.float32) if with_hist else None
    xd = dev(x["qkv"])
    cs = dev(hist.copy()) if with_hist else None
    y = gdn.gdn_conv_silu(xd, dev(x["conv_w"]), cs, l2_channels=2 * Hk * d, head_dim=d,
                          y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    yr, hr = oracle.conv_silu(to_f64(x["qkv"]), to_f64(x["conv_w"]), hist)
    yr = oracle.l2norm_heads(yr.reshape(B * T, C), 2 * Hk * d, d).reshape(B, T, C)
    tol = TOL[ydt]  # the arithmetic is f32; the bar follows the output's rounding
    assert max_rel_err(host_f64(y), yr) < tol
    # Each part separately: q|k heads (normalised) and v.
    assert max_rel_err(host_f64(y)[..., 2 * Hk * d:], yr[..., 2 * Hk * d:]) < tol
    if with_hist:
        assert np.array_equal(host_f64(cs), hr)  # history is copied exactly


def test_conv_split_calls_match_one_call():
    banner("conv_silu split with history carry")
    B, T, C = 1, 200, 1024
    x = mixer_inputs(B, T, Hk=1, Hv=6, d=128, seed=5)
    w = dev(x["conv_w"])
    xd = dev(x["qkv"])
    cs = torch.zeros((B, 3, C), dtype=torch.float32, device="cuda")
    y_full = gdn.gdn_conv_silu(xd, w, cs.clone(), l2_channels=256)
    ys = []
    for t0, t1 in ((0, 1), (1, 3), (3, 67), (67, 200)):
        ys.append(gdn.gdn_conv_silu(xd[:, t0:t1].contiguous(), w, cs, l2_channels=256))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, dim=1), y_full)


@pytest.mark.parametrize("B,T", [(2, 150), (1, 1), (3, 1)])
def test_conv_silu_reads_a_column_range_in_place(B, T):
    """x as the q|k|v columns of a wider [B, T, 16384-like] buffer (the layout
    of one in_proj_qkvz product): bitwise the result of a contiguous copy,
    history included, and within the bar of the oracle."""
    banner(f"conv_silu strided x B={B} T={T}")
    Hk, Hv, d = 2, 6, 128
    C = 2 * Hk * d + Hv * d
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=70 + T)
    rng = np.random.default_rng(71 + T)
    hist = rng.normal(size=(B, 3, C)).astype(np.float32)
    wide = torch.randn((B, T, C + Hv * d + 40), dtype=torch.bfloat16, device="cuda")
    off = 16
    wide[:, :, off:off + C] = dev(x["qkv"])
    xv = wide[:, :, off:off + C]
    assert B * T == 1 or not xv.is_contiguous()
    w = dev(x["conv_w"])
    cs1, cs2 = dev(hist.copy()), dev(hist.copy())
    y1 = gdn.gdn_conv_silu(xv, w, cs1, l2_channels=2 * Hk * d, head_dim=d)
    y2 = gdn.gdn_conv_silu(xv.contiguous(), w, cs2, l2_channels=2 * Hk * d, head_dim=d)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(cs1, cs2)
    yr, hr = oracle.conv_silu(to_f64(x["qkv"]), to_f64(x["conv_w"]), hist)
    yr = oracle.l2norm_heads(yr.reshape(B * T, C), 2 * Hk * d, d).reshape(B, T, C)
    assert max_rel_err(host_f64(y1), yr) < TOL["bf16"]
    assert np.array_equal(host_f64(cs1), hr)


# ------------------------------------------------------------------ gated RMSNorm

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N,H", [(300, 6), (1, 1), (17, 48)])
def test_gated_rmsnorm_parity(dt, N, H):
    banner(f"gated_rmsnorm dt={dt} N={N} H={H}")
    rng = np.random.default_rng(N * 100 + H)
    from synth import bf16_round, f32_round
    rnd = bf16_round if dt == "bf16" else f32_round
    x = rnd(rng.normal(size=(N, H, 128)))
    z = rnd(rng.normal(size=(N, H, 128)))
    w = f32_round(rng.normal(0, 0.1, 128))
    y = gdn.gdn_gated_rmsnorm(dev(x), dev(z), dev(w))
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(to_f64(x), to_f64(z), to_f64(w))
    assert max_rel_err(host_f64(y), ref) < TOL[dt]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_gated_rmsnorm_z_column_range(dt):
    """z as the last Hv*128 columns of a wider buffer, in place (the z part of
    one in_proj_qkvz product): bitwise the result of a contiguous z."""
    banner(f"gated_rmsnorm strided z {dt}")
    N, H = 301, 6
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn((N, H, 128), generator=g).to(dt).cuda()
    wide = torch.randn((N, 1024 + H * 128), generator=g).to(dt).cuda()
    zv = wide[:, 1024:].unflatten(1, (H, 128))
    w = (0.1 * torch.randn(128, generator=g)).cuda()
    y1 = gdn.gdn_gated_rmsnorm(x, zv, w)
    y2 = gdn.gdn_gated_rmsnorm(x, zv.contiguous(), w)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = oracle.gated_rmsnorm(host_f64(x), host_f64(zv.contiguous()), host_f64(w))
    assert max_rel_err(host_f64(y1), ref) < TOL["bf16" if dt == torch.bfloat16 else "f32"]


# ------------------------------------------------------------------ decode_rows

def _decode_ref(x, lengths=None):
    q, k, v = (to_f64(x[n])[:, None] for n in "qkv")   # [R, 1, H, d]
    a, b = to_f64(x["a"])[:, None], to_f64(x["b"])[:, None]
    al, be, _ = oracle.gates(a, b, x["A_log"], x["dt_bias"])
    S0 = to_f64(x["state"])
    o, S = oracle.recurrence(q, k, v, al, be, S0)
    o = o[:, 0]
    if lengths is not None:
        idle = lengths < 0
        o[idle] = 0.0
        S[idle] = S0[idle]
    return o, S


@pytest.mark.parametrize("qdt,gdt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
def test_decode_rows_small(qdt, gdt):
    banner(f"decode_rows small {qdt}/{gdt}")
    x = decode_inputs(5, Hk=2, Hv=6, qkv_dt=qdt, gate_dt=gdt, seed=3)
    st = dev(x["state"])
    o = gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                            dev(x["A_log"]), dev(x["dt_bias"]), st, dev(x["lengths"]))
    torch.cuda.synchronize()
    o_ref, S_ref = _decode_ref(x)
    assert max_rel_err(host_f64(o), o_ref) < TOL[qdt]
    assert max_rel_err(host_f64(st), S_ref) < 1e-5


def test_decode_rows_idle_rows_untouched():
    banner("decode_rows idle rows")
    x = decode_inputs(6, Hk=2, Hv=6, seed=4)
    lengths = x["lengths"].copy()
    lengths[[1, 4]] = -1
    st = dev(x["state"])
    o = gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                            dev(x["A_log"]), dev(x["dt_bias"]), st, dev(lengths))
    torch.cuda.synchronize()
    S = st.cpu().numpy()
    assert np.array_equal(S[[1, 4]], x["state"][[1, 4]])  # bitwise untouched
    assert np.all(host_f64(o)[[1, 4]] == 0.0)
    o_ref, S_ref = _decode_ref(x, lengths)
    assert max_rel_err(host_f64(o), o_ref) < 2e-2
    assert max_rel_err(S.astype(np.float64), S_ref) < 1e-5


def test_decode_rows_workload_r64():
    """decode_rows at its full size: 64 rows, 48 value heads, f32 state."""
    banner("decode_rows_r64 full")
    x = make_workload("decode_rows_r64")
    st = dev(x["state"])
    o = gdn.gdn_decode_rows(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                            dev(x["A_log"]), dev(x["dt_bias"]), st, dev(x["lengths"]))
    torch.cuda.synchronize()
    o_ref, S_ref = _decode_ref(x)
    assert max_rel_err(host_f64(o), o_ref) < 2e-2
    assert max_rel_err(host_f64(st), S_ref) < 1e-5


def test_decode_rows_row_isolation_under_nan():
    banner("decode_rows NaN isolation")
    x = decode_inputs(4, Hk=2, Hv=6, seed=6)
    x2 = {k: (v.copy() if v is not None else None) for k, v in x.items()}
    x2["v"][2, 3, 5] = 0x7FC0  # bf16 NaN in row 2
    outs = []
    for inp in (x, x2):
        st = dev(inp["state"])
        o = gdn.gdn_decode_rows(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]),
                                dev(inp["b"]), dev(inp["A_log"]), dev(inp["dt_bias"]), st)
        torch.cuda.synchronize()
        outs.append((host_f64(o), st.cpu().numpy()))
    keep = [0, 1, 3]
    assert np.array_equal(outs[0][0][keep], outs[1][0][keep])
    assert np.array_equal(outs[0][1][keep], outs[1][1][keep])


# ------------------------------------------------------------------ sequential prefill

def _prefill_ref(x, S0=None):
    q, k, v = (to_f64(x[n]) for n in "qkv")
    al, be, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    return oracle.recurrence(q, k, v, al, be, S0)


def _run_prefill(x, algo, state_in=None, inplace=False):
    si = dev(state_in) if state_in is not None else None
    B, T, Hv = x["v"].shape[0], x["v"].shape[1], x["v"].shape[2]
    so = si if (inplace and si is not None) else torch.empty((B, Hv, 128, 128), dtype=torch.float32,
                                                           device="cuda")
    o = gdn.gdn_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                        dev(x["A_log"]), dev(x["dt_bias"]), si, so, algo=algo)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(so)


def test_prefill_recurrence_f32_b1_t64():
    """The f32 workload: B=1, T=64, 16/48 heads, zero state; tolerance 1e-4."""
    banner("recurrence_f32_b1_t64")
    x = make_workload("recurrence_f32_b1_t64")
    o, S = _run_prefill(x, "auto")
    o_ref, S_ref = _prefill_ref(x)
    assert max_rel_err(o, o_ref) < 1e-4
    assert max_rel_err(S, S_ref) < 1e-4


@pytest.mark.parametrize("qdt,gdt,T,state", [("bf16", "f32", 150, 0.05), ("bf16", "bf16", 1, 0.05),
                                            ("f32", "bf16", 33, None), ("bf16", "f32", 0, 0.05)])
def test_prefill_sequential_small(qdt, gdt, T, state):
    banner(f"prefill sequential {qdt}/{gdt} T={T}")
    x = recurrence_inputs(2, T, Hk=2, Hv=6, qkv_dt=qdt, gate_dt=gdt, seed=T + 1, state_std=state)
    o, S = _run_prefill(x, "sequential", x["state"], inplace=True)
    S0 = None if x["state"] is None else to_f64(x["state"])
    o_ref, S_ref = _prefill_ref(x, S0)
    if T > 0:
        assert max_rel_err(o, o_ref) < TOL[qdt]
    assert max_rel_err(S, S_ref) < 1e-4
