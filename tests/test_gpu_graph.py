"""A whole-layer decode step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give the eager step's results bit for bit.

The step for R fixed rows: in_proj_qkv and in_proj_z as one product with the
stacked weight (gdn_linear into one [R, 16384] buffer), the gate projections
(gdn_gate_proj), the conv over one token with each row's conv history
(gdn_conv_silu, reading the q|k|v columns in place), decode_rows, the gated
RMSNorm in place (reading the z columns in place) and out_proj.
The eager calls run first (they also create the hipBLASLt handle, which may
allocate, and the shapes' plans, so that the captured calls reuse the same
plans as the eager step).  The graph is replayed four
times with eager work and synchronisations in between; before each replay
the captured buffers are reset to the same inputs, so each replay must equal
the eager step exactly.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_mixer_amd as gdn
from synth.inputs import CONV_CH, HIDDEN, HK, HV, D, decode_inputs, mixer_inputs, proj_inputs
from tests.gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def _step(L):
    R = L["x"].shape[0]
    gdn.gdn_linear(L["x"], L["W_qkvz"], y=L["qkvz"], workspace=L["lws"])
    gdn.gdn_gate_proj(L["x"], L["W_a"], L["W_b"], a=L["a"], b=L["b"], workspace=L["gws"])
    gdn.gdn_conv_silu(L["qkv"], L["conv_w"], L["conv_state"], l2_channels=2 * HK * D, y=L["y"])
    y = L["y"][:, 0]
    gdn.gdn_decode_rows(y[:, :HK * D].unflatten(1, (HK, D)),
                        y[:, HK * D:2 * HK * D].unflatten(1, (HK, D)),
                        y[:, 2 * HK * D:].unflatten(1, (HV, D)), L["a"], L["b"], L["A_log"],
                        L["dt_bias"], L["state"], o=L["o"])
    gdn.gdn_gated_rmsnorm(L["o"], L["qkvz"][:, CONV_CH:].unflatten(1, (HV, D)), L["norm_w"],
                          y=L["o"])
    gdn.gdn_linear(L["o"].view(R, HV * D), L["W_out"], y=L["out"], workspace=L["lws"])


def _buffers(R, seed):
    p = proj_inputs(R, seed=seed)
    po = proj_inputs(1, K=HV * D, outs=(("W_out", HIDDEN),), gate_H=0, seed=seed + 1)
    d = decode_inputs(R, seed=seed + 2)
    m = mixer_inputs(1, 4, seed=seed + 3)
    L = {n: dev(p[n]) for n in ("x", "W_a", "W_b")}
    L["W_qkvz"] = torch.cat([dev(p["W_qkv"]), dev(p["W_z"])], dim=0)
    L["W_out"] = dev(po["W_out"])
    L.update({n: dev(d[n]) for n in ("state", "A_log", "dt_bias")})
    L["conv_w"] = dev(m["conv_w"])
    L["norm_w"] = dev(m["norm_w"])
    rng = np.random.default_rng(seed + 4)
    L["conv_state"] = dev((rng.standard_normal((R, 3, CONV_CH)) * 0.5).astype(np.float32))
    L["qkvz"] = torch.empty((R, CONV_CH + HV * D), dtype=torch.bfloat16, device="cuda")
    L["qkv"] = L["qkvz"][:, :CONV_CH].unsqueeze(1)  # [R, 1, 10240] view
    L["a"] = torch.empty((R, HV), dtype=torch.float32, device="cuda")
    L["b"] = torch.empty((R, HV), dtype=torch.float32, device="cuda")
    L["y"] = torch.empty((R, 1, CONV_CH), dtype=torch.bfloat16, device="cuda")
    L["o"] = torch.empty((R, HV, D), dtype=torch.bfloat16, device="cuda")
    L["out"] = torch.empty((R, HIDDEN), dtype=torch.bfloat16, device="cuda")
    L["lws"] = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8, device="cuda")
    L["gws"] = torch.empty(max(gdn.gdn_gate_proj_workspace_bytes(R, HIDDEN, HV), 256),
                           dtype=torch.uint8, device="cuda")
    return L


def test_decode_step_graph_replays_match_eager():
    banner("decode step of the whole layer: graph replays vs eager, 64 rows")
    R = 64
    L = _buffers(R, 90)
    state0 = L["state"].clone()
    cs0 = L["conv_state"].clone()
    _step(L)  # eager; builds the hipBLASLt plans
    torch.cuda.synchronize()
    ref = {n: L[n].clone() for n in ("out", "state", "conv_state", "a", "b", "o", "qkvz")}

    def reset():
        L["state"].copy_(state0)
        L["conv_state"].copy_(cs0)

    reset()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _step(L)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        reset()
        for n in ("out", "a", "b", "o", "qkvz"):
            L[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        scratch.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        for n, r in ref.items():
            assert torch.equal(L[n], r), (rep, n)
