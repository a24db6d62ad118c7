"""The whole mixer path and the long prefill at their full sizes, checked
against the f64 oracle on sampled heads.

Whole mixer, B=4, T=8192 (bf16 in): gdn_conv_silu (10240 channels, width 4,
silu, L2 of q/k, f32 output) -> gdn_prefill (chunked, q/k/v read as strided
views of the conv output, bf16 o) -> gdn_gated_rmsnorm (bf16 y); and the
one-call gdn_mixer_prefill, which must give the same bits (its conv writes v
in bf16, the rounding the chunked prefill applies to an f32 v).  Long
prefill: T=65536 as 16 calls of 4096 with the f32 state handed between them,
against one oracle pass.  Value heads are independent given their q/k head,
so the oracle runs only the sampled (batch, head) pairs end to end.
Bar: 2e-2 (bf16 inputs), max|x-ref|/max|ref| per sampled output.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def run_mixer_gpu(x, B, T, Hk, Hv, d, conv_state=None, S=None):
    C = 2 * Hk * d + Hv * d
    y = gdn.gdn_conv_silu(dev(x["qkv"]), dev(x["conv_w"]), conv_state, l2_channels=2 * Hk * d,
                          head_dim=d, y_dtype=torch.float32)
    q = y[:, :, :Hk * d].unflatten(2, (Hk, d))
    k = y[:, :, Hk * d:2 * Hk * d].unflatten(2, (Hk, d))
    v = y[:, :, 2 * Hk * d:].unflatten(2, (Hv, d))
    if S is None:
        S = torch.zeros((B, Hv, d, d), dtype=torch.float32, device="cuda")
    o = gdn.gdn_prefill(q, k, v, dev(x["a"]), dev(x["b"]), dev(x["A_log"]), dev(x["dt_bias"]),
                        S, S, algo="chunked", o_dtype=torch.bfloat16)
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


def oracle_mixer_heads(x, pairs, Hk, Hv, d):
    """Oracle output of the whole mixer for the listed (batch, value head)
    pairs, stacked along the batch axis (one q/k head per entry)."""
    grp = Hv // Hk
    cols, zs, a_l, b_l, Al, db = [], [], [], [], [], []
    for bb, h in pairs:
        kh = h // grp
        ch = np.r_[kh * d:(kh + 1) * d, (Hk + kh) * d:(Hk + kh + 1) * d,
                   2 * Hk * d + h * d:2 * Hk * d + (h + 1) * d]
        cols.append((bb, ch))
    qkv = np.stack([to_f64(x["qkv"][bb][:, ch]) for bb, ch in cols])       # [P, T, 3d]
    w = np.stack([x["conv_w"][ch] for _, ch in cols])                       # [P, 3d, 4]
    outs, Ss = [], []
    for i, (bb, h) in enumerate(pairs):
        y, S, _ = oracle.mixer(qkv[i:i + 1], w[i], to_f64(x["z"][bb:bb + 1, :, h * d:(h + 1) * d]),
                               to_f64(x["a"][bb:bb + 1, :, h:h + 1]),
                               to_f64(x["b"][bb:bb + 1, :, h:h + 1]), x["A_log"][h:h + 1],
                               x["dt_bias"][h:h + 1], x["norm_w"], 1, 1, d)
        outs.append(y[0])
        Ss.append(S[0, 0])
    return outs, Ss


def test_mixer_small_all_heads():
    banner("mixer small B=2 T=150 Hk=2 Hv=6")
    B, T, Hk, Hv, d = 2, 150, 2, 6, 128
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, seed=31)
    cs = torch.zeros((B, 3, 2 * Hk * d + Hv * d), dtype=torch.float32, device="cuda")
    out, S = run_mixer_gpu(x, B, T, Hk, Hv, d, conv_state=cs)
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                       to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                       x["norm_w"], Hk, Hv, d)
    assert max_rel_err(host_f64(out).reshape(B, T, Hv * d), y_ref) < TOL
    assert max_rel_err(host_f64(S), S_ref) < TOL
    assert np.array_equal(host_f64(cs), h_ref)


@pytest.mark.parametrize("T", [150, 64, 5, 2])
def test_mixer_prefill_one_call_small(T):
    """gdn_mixer_prefill against the oracle, and bitwise against the three
    calls it replaces (with a carried state and conv history)."""
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
    y2, S2 = run_mixer_gpu(x, B, T, Hk, Hv, d, conv_state=cs2, S=S2)
    assert torch.equal(y1.view(B, T, Hv, d), y2)
    assert torch.equal(S1, S2)
    assert torch.equal(cs1, cs2)
    y_ref, S_ref, h_ref = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                       to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                       x["norm_w"], Hk, Hv, d, conv_hist=host_f64(h0),
                                       S0=host_f64(S0))
    assert max_rel_err(host_f64(y1), y_ref) < TOL
    assert max_rel_err(host_f64(S1), S_ref) < TOL
    assert np.array_equal(host_f64(cs1), h_ref)


def test_mixer_prefill_f32_inputs_and_edge_cases():
    """f32 qkv/z/y (the bf16 accuracy class of the chunked path), no conv
    history (NULL: zeros, not written), and T == 0 (state passes through)."""
    banner("mixer_prefill f32 B=1 T=100 Hk=2 Hv=6; T=0")
    B, T, Hk, Hv, d = 1, 100, 2, 6, 128
    x = mixer_inputs(B, T, Hk=Hk, Hv=Hv, d=d, dt="f32", seed=53)
    y, S = run_mixer_fused(x, B, T, Hk, Hv, d, conv_state=None)
    assert y.dtype == torch.float32
    y_ref, S_ref, _ = oracle.mixer(to_f64(x["qkv"]), to_f64(x["conv_w"]), to_f64(x["z"]),
                                   to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"],
                                   x["norm_w"], Hk, Hv, d)
    assert max_rel_err(host_f64(y), y_ref) < TOL
    assert max_rel_err(host_f64(S), S_ref) < TOL
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
def test_mixer_bf16_b4_t8192_sampled_heads():
    """The whole-mixer workload at full size; 6 (batch, head) pairs checked."""
    banner("mixer_bf16_b4_t8192 full")
    B, T = 4, 8192
    x = make_workload("mixer_bf16_b4_t8192")
    cs = torch.zeros((B, 3, 2 * HK * D + HV * D), dtype=torch.float32, device="cuda")
    out, S = run_mixer_gpu(x, B, T, HK, HV, D, conv_state=cs)
    pairs = [(0, 0), (0, 47), (1, 17), (2, 31), (3, 2), (3, 46)]
    outs, Ss = oracle_mixer_heads(x, pairs, HK, HV, D)
    out_h = out.view(B, T, HV, D)
    errs = []
    for (bb, h), yr, Sr in zip(pairs, outs, Ss):
        e_y = max_rel_err(host_f64(out_h[bb, :, h]), yr)
        e_s = max_rel_err(host_f64(S[bb, h]), Sr)
        errs.append((bb, h, e_y, e_s))
    print("mixer_bf16_b4_t8192 (b, h, y err, state err):", errs)
    # Conv history: the last 3 input rows, exactly.
    assert np.array_equal(host_f64(cs), to_f64(x["qkv"][:, -3:, :]))
    assert all(e_y < TOL and e_s < TOL for _, _, e_y, e_s in errs)
    # The one-call path, in the launch configuration the bench times: the same bits.
    del S
    cs2 = torch.zeros_like(cs)
    y2, S2 = run_mixer_fused(x, B, T, HK, HV, D, conv_state=cs2)
    assert torch.equal(y2.view(B, T, HV, D), out)
    assert torch.equal(cs2, cs)


@pytest.mark.slow
def test_prefill_t65536_as_16_calls_sampled_heads():
    """Long prefill: 16 sequential 4096-token calls with the f32 state handed
    between them, against one oracle pass over all 65536 tokens."""
    banner("prefill_bf16_b1_t65536_x16 full")
    x = make_workload("prefill_bf16_b1_t65536_x16")
    T, n_calls = 65536, 16
    L = T // n_calls
    qd, kd, vd, ad, bd = (dev(x[n]) for n in ("q", "k", "v", "a", "b"))
    Al, db = dev(x["A_log"]), dev(x["dt_bias"])
    S = torch.zeros((1, HV, D, D), dtype=torch.float32, device="cuda")
    o = torch.empty((1, T, HV, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, L, HK, HV), dtype=torch.uint8,
                     device="cuda")
    for i in range(n_calls):
        sl = slice(i * L, (i + 1) * L)
        gdn.gdn_prefill(qd[:, sl], kd[:, sl], vd[:, sl], ad[:, sl].contiguous(),
                        bd[:, sl].contiguous(), Al, db, S, S, o=o[:, sl], workspace=ws)
    torch.cuda.synchronize()
    heads = [0, 13, 29, 47]
    grp = HV // HK
    q = np.stack([to_f64(x["q"][0, :, h // grp]) for h in heads])[:, :, None]
    k = np.stack([to_f64(x["k"][0, :, h // grp]) for h in heads])[:, :, None]
    v = np.stack([to_f64(x["v"][0, :, h]) for h in heads])[:, :, None]
    a = np.stack([to_f64(x["a"][0, :, h]) for h in heads])[:, :, None]
    b = np.stack([to_f64(x["b"][0, :, h]) for h in heads])[:, :, None]
    errs = []
    for i, h in enumerate(heads):
        al, be, _ = oracle.gates(a[i:i + 1], b[i:i + 1], x["A_log"][h:h + 1], x["dt_bias"][h:h + 1])
        o_ref, S_ref = oracle.recurrence(q[i:i + 1], k[i:i + 1], v[i:i + 1], al, be)
        errs.append((h, max_rel_err(host_f64(o[0, :, h]), o_ref[0, :, 0]),
                     max_rel_err(host_f64(S[0, h]), S_ref[0, 0])))
    print("prefill_bf16_b1_t65536_x16 (h, o err, state err):", errs)
    assert all(eo < TOL and es < TOL for _, eo, es in errs)
