"""Benchmark of the Gated DeltaNet mixer hot path on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs shaped
like the model's layer (16 q/k heads, 48 value heads, width 128):
  1. the layer prefill at B=1, T=4096: one gdn_mixer_prefill call (conv over
     10240 channels, width 4, silu, L2 of q/k -> chunked prefill with the state
     carried in and out -> gated RMSNorm with z);
  2. gdn_prefill alone on the prefill workload (B=1, T=4096, bf16 q/k/v, f32
     gates, carried state ~N(0, 0.05), chunk 64);
  3. gdn_decode_rows on 64 fixed rows (state [64,48,128,128] f32, in place);
  4. gdn_prefill_slots on a server's ragged batch: 16 fixed rows with
     U{1..1024} new tokens each, bf16, states carried in place;
  5. gdn_decode_rows_multi verifying a 4-token draft on 64 fixed rows, with
     the state after every token written out as a snapshot;
  6. the projections around the mixer at 4096 tokens: in_proj_qkv and
     in_proj_z (gdn_linear, bf16, into one [4096, 16384] buffer), the two
     gate projections with f32 weights (gdn_gate_proj) and out_proj
     (gdn_linear, 6144 -> 5120);
  7. one decode step of the whole layer for 64 fixed rows: in_proj_qkv,
     in_proj_z, the gate projections, the conv over one token with each row's
     conv history, decode_rows, the gated RMSNorm and out_proj;
  8. the same decode step replayed from a HIP graph (captured once per buffer
     set after the warm-up, so the eight launches go out as one).
Each part is timed with HIP events on the stream it runs on.  The timed
region runs each part's K iterations back to back, part after part (so a part
follows its own previous call, not another part's dirty cache lines), and the
inputs of every part rotate over three independent buffer sets so that the
256 MB last-level cache cannot hold a part's working set between its
launches.

Printed: one JSON line.  value = tokens/s of part 2 (the prefill workload);
decode_rows state GB/s and the layer-prefill tokens/s ride along in the same
line, with the roofline of the dominant kernel and the f64 oracle timed on the
host cores as a CPU baseline.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
ROT = 3                       # buffer sets rotated between steps

HK, HV, D, T_PREFILL, R_DECODE = 16, 48, 128, 4096, 64
C_CONV = 2 * HK * D + HV * D
HIDDEN = 5120


def decode_bytes_per_launch(R=R_DECODE, Hk=HK, Hv=HV, d=D, io_bytes=2, gate_bytes=2):
    """Algorithmic HBM bytes of one decode_rows launch: the f32 state read and
    written once, q/k/v/a/b read, o written, lengths read."""
    state = 2 * R * Hv * d * d * 4
    qkv = R * (2 * Hk * d + Hv * d) * io_bytes
    gates = 2 * R * Hv * gate_bytes
    out = R * Hv * d * io_bytes
    return state + qkv + gates + out + R * 4 + 2 * Hv * 4


def prefill_flops_per_launch(T=T_PREFILL, Hv=HV, d=D, C=64):
    """Algorithmic flops of the chunked form per launch: per chunk and value
    head K K^T, Q K^T, W, U~ (2 C^2 d each ... ) and the chain products
    W H, Q H, K^T U (2 C d^2 each) plus P U (2 C^2 d): 2(5 C^2 d + 3 C d^2)."""
    nc = (T + C - 1) // C
    return nc * Hv * 2 * (5 * C * C * d + 3 * C * d * d)


def slots_flops(sx, Hv=HV, d=D, C=64):
    """Dense-tile chunked flops of a ragged batch: each row's chunks (the last
    one padded to 64 tokens) at 2(5C^2 d + 3C d^2) per chunk and value head."""
    import numpy as np
    lens = np.diff(np.asarray(sx["cu_seqlens"], dtype=np.int64))
    chunks = int(((lens + C - 1) // C).sum())
    return chunks * Hv * 2 * (5 * C * C * d + 3 * C * d * d)


def prefill_bytes_per_launch(T=T_PREFILL, Hk=HK, Hv=HV, d=D):
    """Algorithmic HBM bytes of one prefill call: q, k, v read and o written
    (bf16), a, b read (f32), state read and written (f32)."""
    return (2 * T * Hk * d + 2 * T * Hv * d) * 2 + 2 * T * Hv * 4 + 2 * Hv * d * d * 4


def _src_hash(names):
    """Hash of the kernel sources with comments and blank lines removed, so a
    comment-only edit keeps the counters taken on that code valid."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_mixer_amd", "csrc", n)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def _traffic(kernel_key, src_files, launches_bytes_fn=None):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("src_hash") != _src_hash(src_files):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(budget_s=10.0):
    """The f64 oracle (as it stands) on the prefill workload: gates plus the
    token-by-token recurrence over all 48 value heads of B=1, T=4096, on the
    host's cores, repeated while the total stays within about budget_s.
    Returns the JSON object."""
    import numpy as np
    import oracle
    from synth import make_workload, to_f64
    x = make_workload("prefill_bf16_b1_t4096")
    q, k, v = (to_f64(x[n]) for n in "qkv")
    a, b = to_f64(x["a"]), to_f64(x["b"])
    S0 = to_f64(x["state"])
    times = []
    while not times or (sum(times) + times[0] < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        al, be, _ = oracle.gates(a, b, x["A_log"], x["dt_bias"])
        oracle.recurrence(q, k, v, al, be, S0)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    return {"value": round(T_PREFILL / dt, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds_per_pass": round(dt, 4), "passes": len(times),
            "sample": f"whole prefill workload (B=1, T=4096, 48 value heads: f64 gates + "
                      f"sequential recurrence, OpenMP over heads), {len(times)} passes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 256 MiB device-to-device copy "
                         "three times (a kernel of known traffic for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the mixer shards "
              "by heads with no exchange inside it, so multi-GPU figures are not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_mixer_amd as gdn
    from synth import decode_inputs, make_workload, mixer_inputs, recurrence_inputs
    from synth.inputs import proj_inputs
    from synth.torch_io import dev

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    gdn.lib()

    # ---- inputs (seeded; each part's buffers replicated ROT times)
    mx = mixer_inputs(1, T_PREFILL, seed=2003)
    st_layer = recurrence_inputs(1, 1, seed=2004, state_std=0.05)["state"]
    layer = []
    for _ in range(ROT):
        layer.append({
            "qkv": dev(mx["qkv"]), "z": dev(mx["z"]), "a": dev(mx["a"]), "b": dev(mx["b"]),
            "conv_w": dev(mx["conv_w"]), "A_log": dev(mx["A_log"]), "dt_bias": dev(mx["dt_bias"]),
            "norm_w": dev(mx["norm_w"]), "state": dev(st_layer),
            "conv_state": torch.zeros((1, 3, C_CONV), dtype=torch.float32, device="cuda"),
            "out": torch.empty((1, T_PREFILL, HV * D), dtype=torch.bfloat16, device="cuda"),
            "ws": torch.empty(gdn.gdn_mixer_prefill_workspace_bytes(1, T_PREFILL, HK, HV),
                              dtype=torch.uint8, device="cuda"),
        })
    px = make_workload("prefill_bf16_b1_t4096")
    pre = []
    for _ in range(ROT):
        pre.append({n: dev(px[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state")})
        pre[-1]["o"] = torch.empty((1, T_PREFILL, HV, D), dtype=torch.bfloat16, device="cuda")
    dx = make_workload("decode_rows_r64")
    dec = []
    for _ in range(ROT):
        dec.append({n: dev(dx[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state",
                                            "lengths")})
        dec[-1]["o"] = torch.empty((R_DECODE, HV, D), dtype=torch.bfloat16, device="cuda")
    sx = make_workload("prefill_slots_bf16_r16")
    slot_sets = []
    for _ in range(ROT):
        slot_sets.append({n: dev(sx[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                   "state", "cu_seqlens")})
        slot_sets[-1]["ws"] = torch.empty(
            gdn.gdn_prefill_slots_workspace_bytes(16, sx["max_len"], HK, HV), dtype=torch.uint8,
            device="cuda")
        slot_sets[-1]["o"] = torch.empty((sx["q"].shape[0], HV, D), dtype=torch.bfloat16,
                                         device="cuda")
    slot_tokens = int(sx["cu_seqlens"][-1])
    mx4 = make_workload("decode_rows_r64_k4")
    multi = []
    for _ in range(ROT):
        multi.append({n: dev(mx4[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                "state", "lengths")})
        multi[-1]["snap"] = torch.empty((R_DECODE, 4, HV, D, D), dtype=torch.float32,
                                        device="cuda")
        multi[-1]["o"] = torch.empty((R_DECODE, 4, HV, D), dtype=torch.bfloat16, device="cuda")
    pin = proj_inputs(T_PREFILL, seed=2007)
    pout = proj_inputs(T_PREFILL, K=HV * D, outs=(("W_out", HIDDEN),), gate_H=0, seed=2008,
                       x_name="y")
    gws_bytes = max(gdn.gdn_gate_proj_workspace_bytes(T_PREFILL, HIDDEN, HV), 256)
    proj = []
    for _ in range(ROT):
        pj = {n: dev(pin[n]) for n in ("x", "W_qkv", "W_z", "W_a", "W_b")}
        pj.update({"y": dev(pout["y"]), "W_out": dev(pout["W_out"])})
        pj["yin"] = torch.empty((T_PREFILL, C_CONV + HV * D), dtype=torch.bfloat16, device="cuda")
        pj["a"] = torch.empty((T_PREFILL, HV), dtype=torch.float32, device="cuda")
        pj["b"] = torch.empty((T_PREFILL, HV), dtype=torch.float32, device="cuda")
        pj["out"] = torch.empty((T_PREFILL, HIDDEN), dtype=torch.bfloat16, device="cuda")
        pj["lws"] = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8,
                                device="cuda")
        pj["gws"] = torch.empty(gws_bytes, dtype=torch.uint8, device="cuda")
        proj.append(pj)
    del pin, pout
    # Part 7: the layer's decode step for 64 rows (weights shared with part 6).
    dlx = proj_inputs(R_DECODE, outs=(), gate_H=0, seed=2009)["x"]
    dly = decode_inputs(R_DECODE, seed=2010)
    dlayer = []
    for _ in range(ROT):
        dl = {"x": dev(dlx), "state": dev(dly["state"]), "A_log": dev(dly["A_log"]),
              "dt_bias": dev(dly["dt_bias"]), "conv_w": dev(mx["conv_w"]),
              "norm_w": dev(mx["norm_w"]),
              "conv_state": torch.zeros((R_DECODE, 3, C_CONV), dtype=torch.float32,
                                        device="cuda")}
        dl["qkv"] = torch.empty((R_DECODE, 1, C_CONV), dtype=torch.bfloat16, device="cuda")
        dl["z"] = torch.empty((R_DECODE, HV * D), dtype=torch.bfloat16, device="cuda")
        dl["a"] = torch.empty((R_DECODE, HV), dtype=torch.float32, device="cuda")
        dl["b"] = torch.empty((R_DECODE, HV), dtype=torch.float32, device="cuda")
        dl["y"] = torch.empty((R_DECODE, 1, C_CONV), dtype=torch.bfloat16, device="cuda")
        dl["o"] = torch.empty((R_DECODE, HV, D), dtype=torch.bfloat16, device="cuda")
        dl["out"] = torch.empty((R_DECODE, HIDDEN), dtype=torch.bfloat16, device="cuda")
        dl["gws"] = torch.empty(max(gdn.gdn_gate_proj_workspace_bytes(R_DECODE, HIDDEN, HV), 256),
                                dtype=torch.uint8, device="cuda")
        dlayer.append(dl)
    ws_bytes = gdn.gdn_prefill_workspace_bytes(1, T_PREFILL, HK, HV)
    ws = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") for _ in range(ROT)]

    # The parts of a step, each one call.  The timed region runs each part's K
    # iterations back to back (part after part), so a part follows its own
    # previous call rather than another part that left the last-level cache
    # full of its dirty lines; the K steps and their total are the same.
    def layer_part(i):
        L = layer[i % ROT]
        gdn.gdn_mixer_prefill(L["qkv"], L["z"], L["conv_w"], L["a"], L["b"], L["A_log"],
                              L["dt_bias"], L["norm_w"], HK, HV, conv_state=L["conv_state"],
                              state_in=L["state"], state_out=L["state"], y=L["out"],
                              workspace=L["ws"])

    def prefill_part(i):
        P = pre[i % ROT]
        gdn.gdn_prefill(P["q"], P["k"], P["v"], P["a"], P["b"], P["A_log"], P["dt_bias"],
                        P["state"], P["state"], o=P["o"], workspace=ws[i % ROT])

    def decode_part(i):
        Dd = dec[i % ROT]
        gdn.gdn_decode_rows(Dd["q"], Dd["k"], Dd["v"], Dd["a"], Dd["b"], Dd["A_log"],
                            Dd["dt_bias"], Dd["state"], Dd["lengths"], o=Dd["o"])

    def slots_part(i):
        Sx = slot_sets[i % ROT]
        gdn.gdn_prefill_slots(Sx["q"], Sx["k"], Sx["v"], Sx["a"], Sx["b"], Sx["A_log"],
                              Sx["dt_bias"], Sx["cu_seqlens"], Sx["state"], sx["max_len"],
                              o=Sx["o"], workspace=Sx["ws"])

    def multi_part(i):
        M = multi[i % ROT]
        gdn.gdn_decode_rows_multi(M["q"], M["k"], M["v"], M["a"], M["b"], M["A_log"],
                                  M["dt_bias"], M["state"], M["snap"], M["lengths"], o=M["o"])

    # Part 6 records an event after each of its four calls as well.
    proj_ev = {}

    def proj_part(i):
        Pj = proj[i % ROT]
        ev = proj_ev.get(i)
        gdn.gdn_linear(Pj["x"], Pj["W_qkv"], y=Pj["yin"][:, :C_CONV], workspace=Pj["lws"])
        if ev:
            ev[0].record()
        gdn.gdn_linear(Pj["x"], Pj["W_z"], y=Pj["yin"][:, C_CONV:], workspace=Pj["lws"])
        if ev:
            ev[1].record()
        gdn.gdn_gate_proj(Pj["x"], Pj["W_a"], Pj["W_b"], a=Pj["a"], b=Pj["b"],
                          workspace=Pj["gws"])
        if ev:
            ev[2].record()
        gdn.gdn_linear(Pj["y"], Pj["W_out"], y=Pj["out"], workspace=Pj["lws"])

    # Part 7 records an event after each of its first six calls.
    dl_ev = {}

    def dlayer_part(i, events=True):
        L = dlayer[i % ROT]
        W = proj[i % ROT]
        ev = dl_ev.get(i) if events else None
        mark = (lambda j: ev[j].record()) if ev else (lambda j: None)
        gdn.gdn_linear(L["x"], W["W_qkv"], y=L["qkv"].view(R_DECODE, C_CONV), workspace=W["lws"])
        mark(0)
        gdn.gdn_linear(L["x"], W["W_z"], y=L["z"], workspace=W["lws"])
        mark(1)
        gdn.gdn_gate_proj(L["x"], W["W_a"], W["W_b"], a=L["a"], b=L["b"], workspace=L["gws"])
        mark(2)
        gdn.gdn_conv_silu(L["qkv"], L["conv_w"], L["conv_state"], l2_channels=2 * HK * D,
                          y=L["y"])
        mark(3)
        y = L["y"][:, 0]
        gdn.gdn_decode_rows(y[:, :HK * D].unflatten(1, (HK, D)),
                            y[:, HK * D:2 * HK * D].unflatten(1, (HK, D)),
                            y[:, 2 * HK * D:].unflatten(1, (HV, D)), L["a"], L["b"], L["A_log"],
                            L["dt_bias"], L["state"], o=L["o"])
        mark(4)
        gdn.gdn_gated_rmsnorm(L["o"], L["z"].view(R_DECODE, HV, D), L["norm_w"], y=L["o"])
        mark(5)
        gdn.gdn_linear(L["o"].view(R_DECODE, HV * D), W["W_out"], y=L["out"], workspace=W["lws"])

    parts_fn = [layer_part, prefill_part, decode_part, slots_part, multi_part, proj_part,
                dlayer_part]
    for fn in parts_fn:
        for i in range(args.warmup):
            fn(i)
    torch.cuda.synchronize()
    # Part 8: the decode step of each buffer set captured in a graph (the eager
    # warm-up above built the hipBLASLt plans, which cannot be made under capture).
    # A capture that fails leaves part 8 out (graph_us is then null); the
    # replays' results are checked against the eager step in the GPU tests.
    graphs = []
    try:
        cap = torch.cuda.Stream()
        for r in range(ROT):
            gr = torch.cuda.CUDAGraph()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(gr, stream=cap):
                    dlayer_part(r, events=False)
            torch.cuda.current_stream().wait_stream(cap)
            graphs.append(gr)
        torch.cuda.synchronize()
    except RuntimeError as e:
        print(f"bench.py: graph capture of the decode step failed ({e}); part 8 skipped",
              file=sys.stderr)
        graphs = []
        torch.cuda.synchronize()

    def dlayer_graph_part(i):
        graphs[i % ROT].replay()

    if graphs:
        parts_fn.append(dlayer_graph_part)
        for i in range(max(args.warmup, 2)):
            dlayer_graph_part(i)
        torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)] for _ in parts_fn]
    for i in range(args.steps):
        proj_ev[args.warmup + i] = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        dl_ev[args.warmup + i] = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for j, fn in enumerate(parts_fn):
        for i in range(args.steps):
            evs[j][i][0].record()
            fn(args.warmup + i)
            evs[j][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    parts = np.array([[evs[j][i][0].elapsed_time(evs[j][i][1]) for j in range(len(parts_fn))]
                      for i in range(args.steps)])  # ms
    mean = parts.mean(axis=0)
    t_layer, t_pre, t_dec, t_slots, t_multi, t_proj, t_dlayer = mean[:7]
    t_dgraph = mean[7] if len(mean) > 7 else None
    # Per call of part 7: in_proj_qkv, in_proj_z, gates, conv, decode_rows, norm, out_proj.
    dlc = []
    for i in range(args.steps):
        e = [evs[6][i][0]] + dl_ev[args.warmup + i] + [evs[6][i][1]]
        dlc.append([e[j].elapsed_time(e[j + 1]) for j in range(7)])
    dlc = np.array(dlc).mean(axis=0)  # ms
    # Per call of part 6: in_proj_qkv, in_proj_z, gate projections, out_proj.
    pc = np.array([[evs[5][i][0].elapsed_time(proj_ev[args.warmup + i][0]),
                    proj_ev[args.warmup + i][0].elapsed_time(proj_ev[args.warmup + i][1]),
                    proj_ev[args.warmup + i][1].elapsed_time(proj_ev[args.warmup + i][2]),
                    proj_ev[args.warmup + i][2].elapsed_time(evs[5][i][1])]
                   for i in range(args.steps)]).mean(axis=0)  # ms
    t_qkv, t_z, t_gate, t_out = pc
    gemm_flops = 2.0 * T_PREFILL * HIDDEN * (C_CONV + HV * D) + 2.0 * T_PREFILL * HV * D * HIDDEN
    gemm_tflops = gemm_flops / ((t_qkv + t_z + t_out) * 1e-3) / 1e12
    gate_bytes = T_PREFILL * HIDDEN * 2 + 2 * HV * HIDDEN * 4 + 2 * T_PREFILL * HV * 4
    multi_bytes = (2 + 4) * R_DECODE * HV * D * D * 4  # state in + out, 4 snapshots
    ms_per_step = wall * 1e3 / args.steps

    prefill_tps = T_PREFILL / (t_pre * 1e-3)
    layer_tps = T_PREFILL / (t_layer * 1e-3)
    dec_bytes = decode_bytes_per_launch()
    state_bytes = 2 * R_DECODE * HV * D * D * 4
    dec_gbps = state_bytes / (t_dec * 1e-3) / 1e9

    # Rooflines.  The prefill call (two launches: chunk_prep, then chunk_chain)
    # is MFMA work; decode_rows is one HBM-bound launch.  "roofline" is the
    # one that takes more of the step.
    pre_flops = prefill_flops_per_launch()
    ach_d = dec_bytes / (t_dec * 1e-3) / 1e9
    roof_dec = {"bound": "hbm", "kernel": "decode_rows_kernel<bf16,bf16>",
                "achieved": round(ach_d, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach_d / HBM_PEAK_GBPS, 4),
                "traffic": _traffic("decode_rows", ["recurrent.hip", "common.hpp"]),
                "bytes_per_launch": dec_bytes, "avg_launch_us": round(t_dec * 1e3, 2)}
    ach_p = pre_flops / (t_pre * 1e-3) / 1e12
    roof_pre = {"bound": "mfma",
                "kernel": "gdn_prefill chunked: chunk_prep_kernel + chunk_chain_kernel (two launches)",
                "achieved": round(ach_p, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach_p / BF16_MFMA_PEAK_TFLOPS, 4),
                "traffic": _traffic("prefill_chunked", ["chunk_prefill.hip", "chunk_common.hpp", "common.hpp"]),
                "flops_per_launch": pre_flops, "avg_launch_us": round(t_pre * 1e3, 2)}
    roofline, roofline_other = (roof_pre, roof_dec) if t_pre >= t_dec else (roof_dec, roof_pre)

    copy_gbps = None
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for i in range(3):
            ce[i].record()
            dst.copy_(src)
        ce[3].record()
        torch.cuda.synchronize()
        copy_gbps = round(2 * src.numel() * 4 / (ce[1].elapsed_time(ce[3]) / 2 * 1e-3) / 1e9, 1)

    out = {
        "metric": "GDN layer prefill tokens/s (T=4096) + decode_rows state GB/s at 64 rows",
        "value": round(prefill_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_bf16_b1_t4096", "B": 1, "T": T_PREFILL, "chunk": 64,
                   "qk_heads": HK, "v_heads": HV, "head_dim": D,
                   "step": "layer prefill (gdn_mixer_prefill: conv+silu+L2 -> chunked prefill "
                           "-> gated RMSNorm) at B=1 T=4096, prefill workload at B=1 T=4096, "
                           "decode_rows at 64 rows, prefill_slots (16 rows), decode_rows_multi "
                           "(64 rows x 4), projections at 4096 tokens, a 64-row decode step of "
                           "the whole layer (eager and replayed from a HIP graph)"},
        "decode_rows": {"value": round(dec_gbps, 1), "unit": "GB/s (state bytes read+written)",
                        "workload": "decode_rows_r64", "avg_launch_us": round(t_dec * 1e3, 2),
                        "frac_of_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4)},
        "layer_prefill": {"value": round(layer_tps, 1), "unit": "tokens/s",
                          "workload": "gdn_mixer_prefill (conv+silu+L2 -> chunked prefill -> "
                                      "gated RMSNorm), B=1 T=4096, 10240 conv channels",
                          "call_us": round(t_layer * 1e3, 2)},
        "prefill_slots": {"value": round(slot_tokens / (t_slots * 1e-3), 1), "unit": "tokens/s",
                          "workload": "prefill_slots_bf16_r16 (16 fixed rows, U{1..1024} new "
                                      "tokens each, %d tokens, longest %d)" % (slot_tokens,
                                                                                sx["max_len"]),
                          "call_us": round(t_slots * 1e3, 2),
                          "mfma_tflops": round(slots_flops(sx) / (t_slots * 1e-3) / 1e12, 2)},
        "decode_rows_multi": {"value": round(4 * R_DECODE / (t_multi * 1e-3), 1),
                              "unit": "tokens/s",
                              "workload": "decode_rows_r64_k4 (64 rows x 4 draft tokens, state "
                                          "snapshot after every token)",
                              "call_us": round(t_multi * 1e3, 2),
                              "state_gbps": round(multi_bytes / (t_multi * 1e-3) / 1e9, 1)},
        "projections": {
            "workload": "in_proj_qkv 5120->10240 and in_proj_z 5120->6144 (bf16, hipBLASLt), "
                        "in_proj_a/b 5120->48 (f32 weights, gdn_gate_proj), out_proj "
                        "6144->5120 (bf16, hipBLASLt) at 4096 tokens",
            "call_us": round(t_proj * 1e3, 2),
            "in_proj_qkv_us": round(t_qkv * 1e3, 2), "in_proj_z_us": round(t_z * 1e3, 2),
            "gate_proj_us": round(t_gate * 1e3, 2), "out_proj_us": round(t_out * 1e3, 2),
            "gemm_tflops": round(gemm_tflops, 1),
            "gemm_frac_of_bf16_peak": round(gemm_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "gate_proj_gbps_algorithmic": round(gate_bytes / (t_gate * 1e-3) / 1e9, 1)},
        "full_layer_prefill": {
            "value": round(T_PREFILL / ((t_layer + t_proj) * 1e-3), 1), "unit": "tokens/s",
            "workload": "projections (part 6) + gdn_mixer_prefill (part 1) at B=1 T=4096, "
                        "the two parts' times added",
            "us": round((t_layer + t_proj) * 1e3, 2)},
        "full_layer_decode": {
            "value": round(R_DECODE / (t_dlayer * 1e-3), 1), "unit": "tokens/s",
            "workload": "one decode step of the whole layer for 64 fixed rows: in_proj_qkv, "
                        "in_proj_z, gate projections, conv over one token with the rows' conv "
                        "history, decode_rows, gated RMSNorm, out_proj",
            "us": round(t_dlayer * 1e3, 2),
            "graph_us": round(t_dgraph * 1e3, 2) if t_dgraph else None,
            "graph_value": round(R_DECODE / (t_dgraph * 1e-3), 1) if t_dgraph else None,
            "calls_us": dict(zip(["in_proj_qkv", "in_proj_z", "gate_proj", "conv", "decode_rows",
                                  "gated_rmsnorm", "out_proj"],
                                 [round(v * 1e3, 2) for v in dlc]))},
        "prefill": {"avg_launch_us": round(t_pre * 1e3, 2),
                    "mfma_tflops": round(pre_flops / (t_pre * 1e-3) / 1e12, 2),
                    "hbm_gbps_algorithmic": round(prefill_bytes_per_launch() / (t_pre * 1e-3) / 1e9,
                                                  1)},
        "roofline": roofline,
        "roofline_other": roofline_other,
        "copy_256MiB_GBps": copy_gbps,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
