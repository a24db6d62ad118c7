"""GPU parity of the projections around the mixer against the f64 oracle.

The projections ("Qwen/Qwen3.8-27B" architecture viewer, module tree):
in_proj_qkv 5120->10240, in_proj_z 5120->6144 and out_proj 6144->5120 as bf16
linear layers (gdn_linear), in_proj_a / in_proj_b 5120->48 with f32 weights
(gdn_gate_proj; the "qwen38" code-generation page keeps those weights in f32).

Tolerances, as max|y - ref| / max|ref| over the tensor:
* gdn_gate_proj: every product is exact (bf16 x times an exact three-part bf16
  split of each f32 weight) and the sum is f32, so the error is f32 summation
  error, ~1e-7 here; the bound is 2e-6.  A version that rounded the weights to
  bf16 would sit near 1e-3, which the unrounded-weights test separates
  explicitly.
* gdn_linear, f32 output: f32 accumulation of exact bf16 products, bound 2e-5.
* gdn_linear, bf16 output: one rounding to bf16 (2^-9 relative), bound 5e-3.
These hold for both engines behind gdn_linear: the library's MFMA GEMM (its
tiled form for shapes that fill the GPU, its few-row form for M <= 64, as
gdn_linear_kernel reports) and hipBLASLt (the rest).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_mixer_amd as gdn
import oracle
from synth.inputs import HIDDEN, HV, D, CONV_CH, bf16_round, proj_inputs, to_f64
from tests.conftest import max_rel_err
from tests.gpu_util import banner, dev, host_f64

pytestmark = pytest.mark.gpu

TOL_GATE = 2e-6
TOL_LIN_F32 = 2e-5
TOL_LIN_BF16 = 5e-3


def _gate_ref(x, Wa, Wb):
    xf = to_f64(x)
    return oracle.linear(xf, Wa.astype(np.float64)), oracle.linear(xf, Wb.astype(np.float64))


@pytest.mark.parametrize("M", [1, 17, 64, 130, 1100])
def test_gate_proj_parity(M):
    banner(f"gate_proj M={M} K={HIDDEN} H={HV}")
    p = proj_inputs(M, outs=(), seed=20 + M)
    a, b = gdn.gdn_gate_proj(dev(p["x"]), dev(p["W_a"]), dev(p["W_b"]))
    torch.cuda.synchronize()
    ra, rb = _gate_ref(p["x"], p["W_a"], p["W_b"])
    ea, eb = max_rel_err(host_f64(a), ra), max_rel_err(host_f64(b), rb)
    print(f"gate_proj M={M}: a err {ea:.2e}, b err {eb:.2e}")
    assert ea <= TOL_GATE and eb <= TOL_GATE


def test_gate_proj_uses_weights_unrounded():
    """Weights with all 24 significant bits set: the result must match the f64
    product of the f32 weights far more closely than bf16-rounded weights can."""
    banner("gate_proj unrounded weights")
    M, K, H = 64, 1024, 16
    rng = np.random.default_rng(31)
    x = bf16_round(rng.integers(-3, 4, size=(M, K)).astype(np.float64))
    mant = rng.integers(1 << 23, 1 << 24, size=(2, H, K)).astype(np.float64)
    sign = rng.choice([-1.0, 1.0], size=(2, H, K))
    W = (sign * mant * 2.0 ** -30).astype(np.float32)  # exact in f32, not in bf16
    a, b = gdn.gdn_gate_proj(dev(x), dev(W[0]), dev(W[1]))
    torch.cuda.synchronize()
    ra, rb = _gate_ref(x, W[0], W[1])
    rounded = oracle.linear(to_f64(x), to_f64(bf16_round(W[0])))
    e_round = max_rel_err(rounded, ra)
    ea, eb = max_rel_err(host_f64(a), ra), max_rel_err(host_f64(b), rb)
    print(f"gate_proj unrounded: a err {ea:.2e}, b err {eb:.2e}; bf16 weights would give {e_round:.2e}")
    assert e_round > 1e-4
    assert ea <= TOL_GATE and eb <= TOL_GATE
    assert ea < e_round / 100


@pytest.mark.parametrize("M,K", [(77, 128), (1030, 160)])
def test_gate_proj_strided_views_small_K_and_determinism(M, K):
    """x a column slice of a wider buffer, a and b columns of one [M, 2H]
    buffer (row stride 2H), H = 16, K of 4 or 5 k-steps: most waves get an
    empty k-range, the others uneven ones."""
    banner(f"gate_proj strided M={M} K={K} H=16")
    H = 16
    p = proj_inputs(M, K=K + 64, outs=(), gate_H=0, seed=32)
    rng = np.random.default_rng(33)
    Wa = (rng.standard_normal((H, K)) / np.sqrt(K)).astype(np.float32)
    Wb = (rng.standard_normal((H, K)) / np.sqrt(K)).astype(np.float32)
    xw = dev(p["x"])
    x = xw[:, 32:32 + K]
    ab = torch.full((M, 2 * H), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_gate_proj(x, dev(Wa), dev(Wb), a=ab[:, :H], b=ab[:, H:])
    first = ab.clone()
    gdn.gdn_gate_proj(x, dev(Wa), dev(Wb), a=ab[:, :H], b=ab[:, H:])
    torch.cuda.synchronize()
    assert torch.equal(first, ab)
    xs = to_f64(p["x"])[:, 32:32 + K]
    ra = oracle.linear(xs, Wa.astype(np.float64))
    rb = oracle.linear(xs, Wb.astype(np.float64))
    got = host_f64(ab)
    assert max_rel_err(got[:, :H], ra) <= TOL_GATE
    assert max_rel_err(got[:, H:], rb) <= TOL_GATE


@pytest.mark.parametrize("M,K,H", [(1024, 512, 32), (1029, 1024, 64), (2050, 5120, 48)])
def test_gate_proj_many_tokens_lds_path(M, K, H):
    """From 1024 tokens the token tile is staged through LDS; 2H/16 waves move
    its 512 pieces (two per thread at H = 32, one at H = 64), with ragged last
    token tiles."""
    banner(f"gate_proj many tokens M={M} K={K} H={H}")
    p = proj_inputs(M, K=K, outs=(), gate_H=H, seed=80 + H)
    a, b = gdn.gdn_gate_proj(dev(p["x"]), dev(p["W_a"]), dev(p["W_b"]))
    torch.cuda.synchronize()
    ra, rb = _gate_ref(p["x"], p["W_a"], p["W_b"])
    ea, eb = max_rel_err(host_f64(a), ra), max_rel_err(host_f64(b), rb)
    print(f"gate_proj M={M} K={K} H={H}: a err {ea:.2e}, b err {eb:.2e}")
    assert ea <= TOL_GATE and eb <= TOL_GATE


def test_gate_proj_feeds_decode_gates():
    """a and b from gdn_gate_proj drive gdn_decode_rows (f32 gates) exactly as
    the same values copied from the host do."""
    banner("gate_proj -> decode_rows")
    from synth.inputs import decode_inputs
    R = 8
    p = proj_inputs(R, outs=(), seed=34)
    a, b = gdn.gdn_gate_proj(dev(p["x"]), dev(p["W_a"]), dev(p["W_b"]))
    d = decode_inputs(R, qkv_dt="bf16", gate_dt="f32", seed=35)
    outs = []
    for ga, gb in ((a, b), (a.cpu().to("cuda"), b.cpu().to("cuda"))):
        st = dev(d["state"]).clone()
        o = gdn.gdn_decode_rows(dev(d["q"]), dev(d["k"]), dev(d["v"]), ga, gb, dev(d["A_log"]),
                                dev(d["dt_bias"]), st)
        outs.append((o.clone(), st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("M,N,K,out", [(1, 48, 128, torch.float32), (33, 96, 256, torch.float32),
                                       (64, 512, 5120, torch.bfloat16),
                                       (130, 640, 6144, torch.float32),
                                       (257, 1024, 5120, torch.bfloat16)])
def test_linear_parity(M, N, K, out):
    banner(f"linear M={M} N={N} K={K} out={out}")
    p = proj_inputs(M, K=K, outs=(("W", N),), gate_H=0, seed=40 + M)
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    y = gdn.gdn_linear(dev(p["x"]), dev(p["W"]), out_dtype=out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    e = max_rel_err(host_f64(y), ref)
    print(f"linear {M}x{N}x{K} {out}: err {e:.2e}")
    assert e <= (TOL_LIN_F32 if out == torch.float32 else TOL_LIN_BF16)


def test_linear_tune_then_plain_calls():
    """gdn_linear_tune gives the oracle's product and leaves its timed plan for
    the shape: a later gdn_linear call of the same shape repeats it bit for bit."""
    banner("linear tune M=64 N=512 K=5120")
    M, N, K = 64, 512, 5120
    p = proj_inputs(M, K=K, outs=(("W", N),), gate_H=0, seed=45)
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    x, W = dev(p["x"]), dev(p["W"])
    y0 = gdn.gdn_linear(x, W, out_dtype=torch.float32, workspace=ws)
    y1 = gdn.gdn_linear_tune(x, W, out_dtype=torch.float32, workspace=ws)
    y2 = gdn.gdn_linear(x, W, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    for y in (y0, y1, y2):
        assert max_rel_err(host_f64(y), ref) <= TOL_LIN_F32
    assert torch.equal(y1, y2)


def test_linear_many_row_counts():
    """A ragged caller's pattern: 80 different M in a row (more shapes than the
    plan cache keeps), then the first ones again, each against the oracle."""
    banner("linear 80 row counts")
    N, K = 96, 256
    p = proj_inputs(100, K=K, outs=(("W", N),), gate_H=0, seed=46)
    x, W = dev(p["x"]), dev(p["W"])
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    for M in list(range(1, 81)) + [1, 2, 3, 77]:
        y = gdn.gdn_linear(x[:M], W, out_dtype=torch.float32)
        torch.cuda.synchronize()
        e = max_rel_err(host_f64(y), ref[:M])
        assert e <= TOL_LIN_F32, (M, e)


def test_linear_without_workspace_and_strided_output():
    """qkv and z written as column ranges of one [M, 16384] buffer, x a column
    slice of a wider buffer; no workspace."""
    banner("linear strided, no workspace")
    M, K = 96, 512
    p = proj_inputs(M, K=K + 128, outs=(("W1", 256), ("W2", 128)), gate_H=0, seed=50)
    W1 = p["W1"][:, :K].copy()
    W2 = p["W2"][:, :K].copy()
    xw = dev(p["x"])
    x = xw[:, 64:64 + K]
    yb = torch.full((M, 384), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_linear(x, dev(W1), y=yb[:, :256])
    gdn.gdn_linear(x, dev(W2), y=yb[:, 256:])
    torch.cuda.synchronize()
    xs = to_f64(p["x"])[:, 64:64 + K]
    got = host_f64(yb)
    assert max_rel_err(got[:, :256], oracle.linear(xs, to_f64(W1))) <= TOL_LIN_BF16
    assert max_rel_err(got[:, 256:], oracle.linear(xs, to_f64(W2))) <= TOL_LIN_BF16


@pytest.mark.parametrize("M,N,K,out,with_ws", [(64, 10240, 5120, torch.bfloat16, True),
                                                (17, 6144, 5120, torch.float32, False),
                                                (64, 5120, 6144, torch.bfloat16, False),
                                                (33, 5120, 6144, torch.float32, True),
                                                (8, 100, 192, torch.float32, True)])
def test_linear_few_tokens(M, N, K, out, with_ws):
    """The decode-step shapes (at most 64 tokens: the weight-streaming kernel),
    written into columns 32.. of a wider buffer; with a workspace the K range
    is split and the partials summed, without one it is a single pass.  N = 100
    leaves a partial block of outputs; K = 192 is three stages."""
    banner(f"linear few tokens M={M} N={N} K={K} out={out} ws={with_ws}")
    p = proj_inputs(M, K=K, outs=(("W", N),), gate_H=0, seed=70 + M + N % 97)
    ws = (torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
          if with_ws else None)
    width = (N + 64 + 7) // 8 * 8  # row strides are multiples of 8
    yb = torch.full((M, width), float("nan"), dtype=out, device="cuda")
    gdn.gdn_linear(dev(p["x"]), dev(p["W"]), y=yb[:, 32:32 + N], workspace=ws)
    torch.cuda.synchronize()
    got = host_f64(yb)
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    e = max_rel_err(got[:, 32:32 + N], ref)
    print(f"linear few tokens {M}x{N}x{K}: err {e:.2e}")
    assert e <= (TOL_LIN_F32 if out == torch.float32 else TOL_LIN_BF16)
    assert np.isnan(got[:, :32]).all() and np.isnan(got[:, 32 + N:]).all()


def _sampled_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, size=n, replace=False))


def test_in_proj_full_size_sampled_rows():
    """in_proj_qkv and in_proj_z at B=1 T=4096 (M=4096, K=5120, N=10240 and
    6144) into one [4096, 16384] buffer, plus the gate projections; 48 rows
    checked against the oracle, every column."""
    banner("in_proj full size M=4096")
    M = 4096
    p = proj_inputs(M, seed=60)
    x = dev(p["x"])
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    y = torch.empty(M, CONV_CH + HV * D, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_linear(x, dev(p["W_qkv"]), y=y[:, :CONV_CH], workspace=ws)
    gdn.gdn_linear(x, dev(p["W_z"]), y=y[:, CONV_CH:], workspace=ws)
    a, b = gdn.gdn_gate_proj(x, dev(p["W_a"]), dev(p["W_b"]))
    torch.cuda.synchronize()
    rows = _sampled_rows(M, 48, 61)
    xs = to_f64(p["x"][rows])
    got = host_f64(y[torch.from_numpy(rows).cuda()])
    e1 = max_rel_err(got[:, :CONV_CH], oracle.linear(xs, to_f64(p["W_qkv"])))
    e2 = max_rel_err(got[:, CONV_CH:], oracle.linear(xs, to_f64(p["W_z"])))
    ra, rb = _gate_ref(p["x"][rows], p["W_a"], p["W_b"])
    idx = torch.from_numpy(rows).cuda()
    ea, eb = max_rel_err(host_f64(a[idx]), ra), max_rel_err(host_f64(b[idx]), rb)
    print(f"in_proj full: qkv {e1:.2e}, z {e2:.2e}, a {ea:.2e}, b {eb:.2e}")
    assert e1 <= TOL_LIN_BF16 and e2 <= TOL_LIN_BF16
    assert ea <= TOL_GATE and eb <= TOL_GATE


def test_out_proj_full_size_sampled_rows():
    """out_proj at M=4096, K=6144, N=5120; 48 rows checked, every column."""
    banner("out_proj full size M=4096")
    M = 4096
    p = proj_inputs(M, K=HV * D, outs=(("W_out", HIDDEN),), gate_H=0, seed=62)
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    y = gdn.gdn_linear(dev(p["x"]), dev(p["W_out"]), workspace=ws)
    torch.cuda.synchronize()
    rows = _sampled_rows(M, 48, 63)
    got = host_f64(y[torch.from_numpy(rows).cuda()])
    e = max_rel_err(got, oracle.linear(to_f64(p["x"][rows]), to_f64(p["W_out"])))
    print(f"out_proj full: {e:.2e}")
    assert e <= TOL_LIN_BF16


# Shapes that the library's GEMM takes on a 256-CU MI355X, one per block width
# (x rows in blocks of 256: 2048 or 2000 rows give 8 blocks; the width makes
# N / width * 8 >= 256 tiles), K small enough for the oracle.
OWN_CASES = [(2048, 10240, 512, torch.float32, 320),
             (2000, 10240, 256, torch.bfloat16, 320),   # last x block 208 rows
             (2048, 8192, 256, torch.float32, 256),
             (2048, 6144, 320, torch.bfloat16, 192),
             (2048, 5120, 384, torch.float32, 160),
             (1900, 5120, 128, torch.bfloat16, 160)]    # one k stage pair, ragged M


@pytest.mark.parametrize("M,N,K,out,width", OWN_CASES)
def test_linear_own_gemm_widths(M, N, K, out, width):
    """Each block width of the library's GEMM against the oracle, with ragged
    x-row blocks; two calls give the same bits."""
    banner(f"linear own GEMM M={M} N={N} K={K} out={out} width {width}")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the width choice below assumes 256 CUs")
    assert gdn.gdn_linear_kernel(M, N, K) == width
    p = proj_inputs(M, K=K, outs=(("W", N),), gate_H=0, seed=60 + K)
    x, W = dev(p["x"]), dev(p["W"])
    y = gdn.gdn_linear(x, W, out_dtype=out)
    y2 = gdn.gdn_linear(x, W, out_dtype=out)
    torch.cuda.synchronize()
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    e = max_rel_err(host_f64(y), ref)
    print(f"linear own {M}x{N}x{K} {out} width {width}: err {e:.2e}")
    assert e <= (TOL_LIN_F32 if out == torch.float32 else TOL_LIN_BF16)
    assert torch.equal(y, y2)


def test_linear_own_gemm_strided_and_tuned():
    """The library's GEMM on a column slice of x (x_ld > K) writing columns of a
    wider y (y_ld > N), canaries around y untouched; then gdn_linear_tune on
    the same shape, and a plain call after it repeating the tuned result bit
    for bit, all against the oracle."""
    M, N, K = 2048, 6144, 256
    banner(f"linear own GEMM strided M={M} N={N} K={K}")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the width choice below assumes 256 CUs")
    p = proj_inputs(M, K=K + 64, outs=(("W", N),), gate_H=0, seed=71)
    Wk = dev(p["W"][:, :K].copy())
    xw = dev(p["x"])
    x = xw[:, 32:32 + K]
    assert gdn.gdn_linear_kernel(M, N, K, x_ld=K + 64) == 192
    yb = torch.full((M, N + 64), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_linear(x, Wk, y=yb[:, 32:32 + N])
    torch.cuda.synchronize()
    ref = oracle.linear(to_f64(p["x"])[:, 32:32 + K], to_f64(p["W"][:, :K]))
    got = host_f64(yb)
    assert np.isnan(got[:, :32]).all() and np.isnan(got[:, 32 + N:]).all()
    assert max_rel_err(got[:, 32:32 + N], ref) <= TOL_LIN_F32
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    y1 = gdn.gdn_linear_tune(x, Wk, out_dtype=torch.float32, workspace=ws)
    y2 = gdn.gdn_linear(x, Wk, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert max_rel_err(host_f64(y1), ref) <= TOL_LIN_F32
    assert torch.equal(y1, y2)


def test_linear_kernel_choice_for_the_projections():
    """At 4096 tokens the projections take the library's tiled GEMM (320, 192,
    320 and, for the stacked in_proj_qkvz weight, 256 wide); at 64 decode rows
    its few-row form, split over K where the workspace allows; without a
    workspace only the shapes that need no split stay there."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the width choice below assumes 256 CUs")
    assert gdn.gdn_linear_kernel(4096, 10240, 5120) == 320
    assert gdn.gdn_linear_kernel(4096, 6144, 5120) == 192
    assert gdn.gdn_linear_kernel(4096, 5120, 6144) == 320
    assert gdn.gdn_linear_kernel(4096, 16384, 5120) == 256
    for N, K in ((10240, 5120), (6144, 5120), (5120, 6144), (16384, 5120)):
        assert gdn.gdn_linear_kernel(64, N, K) == 64
    assert gdn.gdn_linear_kernel(64, 16384, 5120, workspace_bytes=0) == 64  # one K range
    assert gdn.gdn_linear_kernel(64, 5120, 6144, workspace_bytes=0) == 0    # needs a split
    assert gdn.gdn_linear_kernel(65, 16384, 5120) == 0     # more than 64 rows
    assert gdn.gdn_linear_kernel(64, 1024, 512) == 0       # too few weight blocks
    assert gdn.gdn_linear_kernel(4096, 10240, 5100) == 0   # K not a multiple of 64


# Shapes the few-row form takes on a 256-CU MI355X (64-row weight blocks times
# equal K ranges >= 192 workgroups): (M, N, K, out dtype, K ranges).
FEWROW_CASES = [(64, 16384, 512, torch.bfloat16, 1),
                (5, 16384, 1024, torch.float32, 1),
                (1, 12288, 256, torch.float32, 1),
                (33, 5120, 1536, torch.float32, 3),     # ragged rows, three ranges
                (64, 4096, 2048, torch.bfloat16, 4)]


@pytest.mark.parametrize("M,N,K,out,splits", FEWROW_CASES)
def test_linear_fewrow_gemm(M, N, K, out, splits):
    """The few-row form against the oracle, x a column slice of a wider buffer
    and y columns of a wider one with canaries around; two calls give the same
    bits (the K ranges' partial sums are added in a fixed order)."""
    banner(f"linear few-row GEMM M={M} N={N} K={K} out={out} ranges {splits}")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the engine choice below assumes 256 CUs")
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    assert gdn.gdn_linear_kernel(M, N, K, x_ld=K + 64) == 64
    if splits > 1:
        assert gdn.gdn_linear_kernel(M, N, K, x_ld=K + 64, workspace_bytes=0) == 0
    p = proj_inputs(M, K=K + 64, outs=(("W", N),), gate_H=0, seed=80 + K)
    Wk = dev(p["W"][:, :K].copy())
    x = dev(p["x"])[:, 64:]
    ys = []
    for _ in range(2):
        yb = torch.full((M, N + 64), float("nan"), dtype=out, device="cuda")
        gdn.gdn_linear(x, Wk, y=yb[:, 64:], workspace=ws)
        ys.append(yb)
    torch.cuda.synchronize()
    got = host_f64(ys[0])
    assert np.isnan(got[:, :64]).all()
    ref = oracle.linear(to_f64(p["x"])[:, 64:], to_f64(p["W"][:, :K]))
    e = max_rel_err(got[:, 64:], ref)
    print(f"linear few-row {M}x{N}x{K} {out} ranges {splits}: err {e:.2e}")
    assert e <= (TOL_LIN_F32 if out == torch.float32 else TOL_LIN_BF16)
    assert torch.equal(ys[0][:, 64:], ys[1][:, 64:])


@pytest.mark.parametrize("N,K", [(16384, 5120), (5120, 6144)])
def test_linear_fewrow_decode_projections_full_size(N, K):
    """The decode step's in_proj_qkvz and out_proj at 64 rows on the few-row
    form (one and three K ranges), every output against the oracle; then
    gdn_linear_tune on the same shape agrees with the oracle too."""
    banner(f"linear few-row full size M=64 N={N} K={K}")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the engine choice below assumes 256 CUs")
    assert gdn.gdn_linear_kernel(64, N, K) == 64
    p = proj_inputs(64, K=K, outs=(("W", N),), gate_H=0, seed=90 + N)
    ws = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    x, W = dev(p["x"]), dev(p["W"])
    y = gdn.gdn_linear(x, W, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.linear(to_f64(p["x"]), to_f64(p["W"]))
    e = max_rel_err(host_f64(y), ref)
    yt = gdn.gdn_linear_tune(x, W, workspace=ws)
    torch.cuda.synchronize()
    et = max_rel_err(host_f64(yt), ref)
    print(f"few-row 64x{N}x{K}: err {e:.2e}; tuned {et:.2e}")
    assert e <= TOL_LIN_BF16 and et <= TOL_LIN_BF16
