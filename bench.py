"""Benchmark of the Gated DeltaNet mixer hot path on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs shaped
like the model's layer (16 q/k heads, 48 value heads, width 128), part by part:
  layer     the layer prefill at B=1, T=4096: one gdn_mixer_prefill call (conv
            over 10240 channels, width 4, silu, L2 of q/k -> chunked prefill
            with the state carried in and out -> gated RMSNorm with z), qkv
            and z read in place as the two column ranges of one [4096, 16384]
            buffer, the layout the fused in_proj_qkvz product writes;
  prefill   gdn_prefill alone on the prefill workload (B=1, T=4096, bf16
            q/k/v, f32 gates, carried state ~N(0, 0.05), chunk 64): the
            headline;
  decode    gdn_decode_rows on 64 fixed rows (state [64,48,128,128] f32, in
            place);
  mixer_b4  the whole-mixer workload: one gdn_mixer_prefill call at B=4,
            T=8192 (bf16, zero initial states);
  long      the long prefill: T=65536 as 16 gdn_prefill calls of 4096 tokens
            with the f32 state handed from call to call;
  slots     gdn_prefill_slots on a server's ragged batch: 16 fixed rows with
            U{1..1024} new tokens each, bf16, states carried in place;
  multi     gdn_decode_rows_multi verifying a 4-token draft on 64 fixed rows,
            with the state after every token written out as a snapshot;
  proj      the projections around the mixer at 4096 tokens: in_proj_qkv and
            in_proj_z as one product with the stacked [16384, 5120] weight
            (gdn_linear, bf16, into one [4096, 16384] buffer), the two gate
            projections with f32 weights (gdn_gate_proj) and out_proj
            (gdn_linear, 6144 -> 5120);
  dlayer    one decode step of the whole layer for 64 fixed rows: the fused
            in_proj_qkvz product, the gate projections, the conv over one
            token with each row's conv history (reading the q|k|v columns in
            place), decode_rows, the gated RMSNorm (reading the z columns in
            place) and out_proj;
  dgraph    the same decode step replayed from a HIP graph (captured once per
            buffer set after the warm-up, so the eight launches go out as one).
Each part is timed with HIP events on the stream it runs on.  The timed
region runs each part's K iterations back to back, part after part (so a part
follows its own previous call, not another part's dirty cache lines), and
every rate uses the region's mean per call; a second pass with events around
each call adds the median, min, p90 and mean of the K calls.  The inputs,
outputs and workspace of every part rotate over three
independent buffer sets so that the 256 MB last-level cache cannot hold a
part's working set between its launches.

Printed: one JSON line.  value = tokens/s of the prefill part (gdn_prefill on
the B=1 T=4096 prefill workload, the chunked gated delta rule alone); the
other parts ride in the same line, with the roofline of the dominant kernel
(the chunked prefill's two launches), the rooflines of the others, a plain
256 MiB copy as the measured HBM reference, and the f64 oracle timed on the
host cores (all cores, and one core on a sample of heads) as a CPU baseline.
--parts selects parts for per-workload profiles (value is then null unless
the prefill part runs).
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


# Sources of the whole mixer's kernels (conv, prep, chain, norm) and of the
# call that sequences them.
MIXER_SRC = ["conv_silu.hip", "chunk_prefill.hip", "chunk_common.hpp", "gated_rmsnorm.hip",
             "common.hpp", "api.hip"]


def mixer_bytes(B, T, Hk=HK, Hv=HV, d=D, io=2):
    """Algorithmic HBM bytes of the whole mixer at B x T (bf16 in and out,
    zero initial state): the fused minimum reads qkv and z, reads a and b,
    writes y and the final state; the unfused chain also writes and re-reads
    the conv output and the recurrence output o.  Returns (fused, unfused)."""
    C = 2 * Hk * d + Hv * d
    qkv, z, y = B * T * C * io, B * T * Hv * d * io, B * T * Hv * d * io
    gates = 2 * B * T * Hv * io
    state = B * Hv * d * d * 4
    fused = qkv + z + y + gates + state
    return fused, fused + 2 * qkv + 2 * y


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=10.0, single_budget_s=4.0, sample_heads=12):
    """The f64 oracle (as it stands) on the prefill workload: gates plus the
    token-by-token recurrence over all 48 value heads of B=1, T=4096, on all
    the host's cores (OpenMP over heads), repeated while the total stays
    within about budget_s; then on one core over the first sample_heads value
    heads (sample_heads/3 q/k heads), scaled to the whole workload (the
    heads are independent and equal work).  Returns the JSON object."""
    import numpy as np
    import oracle
    from synth import make_workload, to_f64
    x = make_workload("prefill_bf16_b1_t4096")
    q, k, v = (to_f64(x[n]) for n in "qkv")
    a, b = to_f64(x["a"]), to_f64(x["b"])
    S0 = to_f64(x["state"])
    cores = oracle.num_threads()

    def run(q, k, v, a, b, Al, db, S0, budget):
        times = []
        while not times or (sum(times) + times[0] < budget and len(times) < 50):
            t0 = time.perf_counter()
            al, be, _ = oracle.gates(a, b, Al, db)
            oracle.recurrence(q, k, v, al, be, S0)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    dt, n = run(q, k, v, a, b, x["A_log"], x["dt_bias"], S0, budget_s)
    g = HV // HK
    nh = sample_heads
    oracle.set_num_threads(1)
    try:
        dt1, n1 = run(q[:, :, :nh // g], k[:, :, :nh // g], v[:, :, :nh], a[:, :, :nh],
                      b[:, :, :nh], x["A_log"][:nh], x["dt_bias"][:nh], S0[:, :nh],
                      single_budget_s)
    finally:
        oracle.set_num_threads(cores)
    t1_whole = dt1 * HV / nh
    return {"value": round(T_PREFILL / dt, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "seconds_per_pass": round(dt, 4), "passes": n,
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"whole prefill workload (B=1, T=4096, 48 value heads: f64 gates + "
                      f"sequential recurrence, OpenMP over heads), median of {n} passes",
            "single_core": {"value": round(T_PREFILL / t1_whole, 1), "unit": "tokens/s",
                            "cores": 1, "seconds_per_pass_sample": round(dt1, 4), "passes": n1,
                            "sample": f"first {nh} of 48 value heads of the same workload on "
                                      f"one thread, median of {n1} passes, scaled by 48/{nh}"}}


PARTS = ("layer", "prefill", "decode", "mixer_b4", "long", "slots", "multi", "proj", "dlayer",
         "dgraph")


def stats(ms):
    """median / min / p90 / mean of per-call times (ms in, us out)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "min_us": round(float(a.min()), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "mean_us": round(float(a.mean()), 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-calibration", action="store_true",
                    help="skip the plain 256 MiB device-to-device copy timed after the steps "
                         "(the measured HBM reference, and a kernel of known traffic for "
                         "scaling HBM counters)")
    ap.add_argument("--parts", default=",".join(PARTS),
                    help="comma-separated parts to run (for per-workload profiles); default all")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the mixer shards "
              "by heads with no exchange inside it, so multi-GPU figures are not measured here.",
              file=sys.stderr)
        sys.exit(2)
    want = [p.strip() for p in args.parts.split(",") if p.strip()]
    bad = [p for p in want if p not in PARTS]
    if bad:
        print(f"unknown parts {bad}; known: {','.join(PARTS)}", file=sys.stderr)
        sys.exit(2)
    if "dgraph" in want and "dlayer" not in want:
        want.append("dlayer")  # the graph replays the decode step's buffers

    import numpy as np
    import torch

    import gated_deltanet_mixer_amd as gdn
    from synth import decode_inputs, make_workload, mixer_inputs, recurrence_inputs
    from synth.inputs import proj_inputs
    from synth.torch_io import dev

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    gdn.lib()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    fns = {}  # part -> fn(i)

    # ---- inputs (seeded; each part's buffers replicated ROT times)
    if "layer" in want:
        mx = mixer_inputs(1, T_PREFILL, seed=2003)
        st_layer = recurrence_inputs(1, 1, seed=2004, state_std=0.05)["state"]
        layer = []
        for _ in range(ROT):
            qkvz = torch.cat([dev(mx["qkv"]), dev(mx["z"])], dim=2)  # [1, T, 16384]
            layer.append({
                "qkv": qkvz[..., :C_CONV], "z": qkvz[..., C_CONV:], "a": dev(mx["a"]),
                "b": dev(mx["b"]),
                "conv_w": dev(mx["conv_w"]), "A_log": dev(mx["A_log"]),
                "dt_bias": dev(mx["dt_bias"]), "norm_w": dev(mx["norm_w"]),
                "state": dev(st_layer),
                "conv_state": torch.zeros((1, 3, C_CONV), dtype=torch.float32, device="cuda"),
                "out": torch.empty((1, T_PREFILL, HV * D), dtype=torch.bfloat16, device="cuda"),
                "ws": torch.empty(gdn.gdn_mixer_prefill_workspace_bytes(1, T_PREFILL, HK, HV),
                                  dtype=torch.uint8, device="cuda"),
            })

        def layer_part(i):
            L = layer[i % ROT]
            gdn.gdn_mixer_prefill(L["qkv"], L["z"], L["conv_w"], L["a"], L["b"], L["A_log"],
                                  L["dt_bias"], L["norm_w"], HK, HV, conv_state=L["conv_state"],
                                  state_in=L["state"], state_out=L["state"], y=L["out"],
                                  workspace=L["ws"])
        fns["layer"] = layer_part

    if "prefill" in want:
        px = make_workload("prefill_bf16_b1_t4096")
        ws_bytes = gdn.gdn_prefill_workspace_bytes(1, T_PREFILL, HK, HV)
        pre = []
        for _ in range(ROT):
            pre.append({n: dev(px[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                "state")})
            pre[-1]["o"] = torch.empty((1, T_PREFILL, HV, D), dtype=torch.bfloat16,
                                       device="cuda")
            pre[-1]["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

        def prefill_part(i):
            P = pre[i % ROT]
            gdn.gdn_prefill(P["q"], P["k"], P["v"], P["a"], P["b"], P["A_log"], P["dt_bias"],
                            P["state"], P["state"], o=P["o"], workspace=P["ws"])
        fns["prefill"] = prefill_part

    if "decode" in want:
        dx = make_workload("decode_rows_r64")
        dec = []
        for _ in range(ROT):
            dec.append({n: dev(dx[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                "state", "lengths")})
            dec[-1]["o"] = torch.empty((R_DECODE, HV, D), dtype=torch.bfloat16, device="cuda")

        def decode_part(i):
            Dd = dec[i % ROT]
            gdn.gdn_decode_rows(Dd["q"], Dd["k"], Dd["v"], Dd["a"], Dd["b"], Dd["A_log"],
                                Dd["dt_bias"], Dd["state"], Dd["lengths"], o=Dd["o"])
        fns["decode"] = decode_part

    B3, T3 = 4, 8192
    if "mixer_b4" in want:
        log("inputs: mixer_bf16_b4_t8192")
        m3 = make_workload("mixer_bf16_b4_t8192")
        m3d = {n: dev(m3[n]) for n in ("qkv", "z", "a", "b", "conv_w", "A_log", "dt_bias",
                                       "norm_w")}
        del m3
        ws3 = gdn.gdn_mixer_prefill_workspace_bytes(B3, T3, HK, HV)
        mix4 = []
        for r in range(ROT):
            M = {n: (t if r == 0 else t.clone()) for n, t in m3d.items()}
            M["state"] = torch.zeros((B3, HV, D, D), dtype=torch.float32, device="cuda")
            M["conv_state"] = torch.zeros((B3, 3, C_CONV), dtype=torch.float32, device="cuda")
            M["out"] = torch.empty((B3, T3, HV * D), dtype=torch.bfloat16, device="cuda")
            M["ws"] = torch.empty(ws3, dtype=torch.uint8, device="cuda")
            mix4.append(M)

        def mixer_b4_part(i):
            M = mix4[i % ROT]
            # zero initial recurrent state (state_in NULL), as the workload has;
            # the conv history is read and rewritten (3 rows per batch row),
            # so a set's later calls start from its previous history: the
            # same work
            gdn.gdn_mixer_prefill(M["qkv"], M["z"], M["conv_w"], M["a"], M["b"], M["A_log"],
                                  M["dt_bias"], M["norm_w"], HK, HV, conv_state=M["conv_state"],
                                  state_in=None, state_out=M["state"], y=M["out"],
                                  workspace=M["ws"])
        fns["mixer_b4"] = mixer_b4_part

    T4, N4 = 65536, 16
    L4 = T4 // N4
    if "long" in want:
        log("inputs: prefill_bf16_b1_t65536_x16")
        lx = make_workload("prefill_bf16_b1_t65536_x16")
        lxd = {n: dev(lx[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
        del lx
        ws4 = gdn.gdn_prefill_workspace_bytes(1, L4, HK, HV)
        longs = []
        for r in range(ROT):
            Lg = {n: (t if r == 0 else t.clone()) for n, t in lxd.items()}
            Lg["state"] = torch.zeros((1, HV, D, D), dtype=torch.float32, device="cuda")
            Lg["o"] = torch.empty((1, T4, HV, D), dtype=torch.bfloat16, device="cuda")
            Lg["ws"] = torch.empty(ws4, dtype=torch.uint8, device="cuda")
            Lg["calls"] = [(Lg["q"][:, c * L4:(c + 1) * L4], Lg["k"][:, c * L4:(c + 1) * L4],
                            Lg["v"][:, c * L4:(c + 1) * L4], Lg["a"][:, c * L4:(c + 1) * L4],
                            Lg["b"][:, c * L4:(c + 1) * L4], Lg["o"][:, c * L4:(c + 1) * L4])
                           for c in range(N4)]
            longs.append(Lg)

        def long_part(i):
            Lg = longs[i % ROT]
            for c, (q, k, v, a, b, o) in enumerate(Lg["calls"]):
                # call 0 starts from the zero state (state_in NULL), the others
                # continue from the state the previous call left
                gdn.gdn_prefill(q, k, v, a, b, Lg["A_log"], Lg["dt_bias"],
                                None if c == 0 else Lg["state"], Lg["state"], o=o,
                                workspace=Lg["ws"])
        fns["long"] = long_part

    if "slots" in want:
        sx = make_workload("prefill_slots_bf16_r16")
        slot_sets = []
        for _ in range(ROT):
            slot_sets.append({n: dev(sx[n]) for n in ("q", "k", "v", "a", "b", "A_log",
                                                       "dt_bias", "state", "cu_seqlens")})
            slot_sets[-1]["ws"] = torch.empty(
                gdn.gdn_prefill_slots_workspace_bytes(16, sx["max_len"], HK, HV),
                dtype=torch.uint8, device="cuda")
            slot_sets[-1]["o"] = torch.empty((sx["q"].shape[0], HV, D), dtype=torch.bfloat16,
                                             device="cuda")
        slot_tokens = int(sx["cu_seqlens"][-1])

        def slots_part(i):
            Sx = slot_sets[i % ROT]
            gdn.gdn_prefill_slots(Sx["q"], Sx["k"], Sx["v"], Sx["a"], Sx["b"], Sx["A_log"],
                                  Sx["dt_bias"], Sx["cu_seqlens"], Sx["state"], sx["max_len"],
                                  o=Sx["o"], workspace=Sx["ws"])
        fns["slots"] = slots_part

    if "multi" in want:
        mx4 = make_workload("decode_rows_r64_k4")
        multi = []
        for _ in range(ROT):
            multi.append({n: dev(mx4[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                    "state", "lengths")})
            multi[-1]["snap"] = torch.empty((R_DECODE, 4, HV, D, D), dtype=torch.float32,
                                            device="cuda")
            multi[-1]["o"] = torch.empty((R_DECODE, 4, HV, D), dtype=torch.bfloat16,
                                         device="cuda")

        def multi_part(i):
            M = multi[i % ROT]
            gdn.gdn_decode_rows_multi(M["q"], M["k"], M["v"], M["a"], M["b"], M["A_log"],
                                      M["dt_bias"], M["state"], M["snap"], M["lengths"],
                                      o=M["o"])
        fns["multi"] = multi_part

    proj_ev, dl_ev = {}, {}
    if "proj" in want or "dlayer" in want:
        mxc = mixer_inputs(1, 1, seed=2003)  # conv and norm weights of the decode step
        pin = proj_inputs(T_PREFILL, seed=2007)
        pout = proj_inputs(T_PREFILL, K=HV * D, outs=(("W_out", HIDDEN),), gate_H=0, seed=2008,
                           x_name="y")
        gws_bytes = max(gdn.gdn_gate_proj_workspace_bytes(T_PREFILL, HIDDEN, HV), 256)
        proj = []
        for _ in range(ROT):
            pj = {n: dev(pin[n]) for n in ("x", "W_a", "W_b")}
            # in_proj_qkv and in_proj_z stacked: one [16384, 5120] weight
            pj["W_qkvz"] = torch.cat([dev(pin["W_qkv"]), dev(pin["W_z"])], dim=0)
            pj.update({"y": dev(pout["y"]), "W_out": dev(pout["W_out"])})
            pj["yin"] = torch.empty((T_PREFILL, C_CONV + HV * D), dtype=torch.bfloat16,
                                    device="cuda")
            pj["a"] = torch.empty((T_PREFILL, HV), dtype=torch.float32, device="cuda")
            pj["b"] = torch.empty((T_PREFILL, HV), dtype=torch.float32, device="cuda")
            pj["out"] = torch.empty((T_PREFILL, HIDDEN), dtype=torch.bfloat16, device="cuda")
            pj["lws"] = torch.empty(gdn.gdn_linear_workspace_bytes(), dtype=torch.uint8,
                                    device="cuda")
            pj["gws"] = torch.empty(gws_bytes, dtype=torch.uint8, device="cuda")
            proj.append(pj)
        del pin, pout

    if "proj" in want:
        # Records an event after each of its first two calls as well.
        def proj_part(i):
            Pj = proj[i % ROT]
            ev = proj_ev.get(i)
            gdn.gdn_linear(Pj["x"], Pj["W_qkvz"], y=Pj["yin"], workspace=Pj["lws"])
            if ev:
                ev[0].record()
            gdn.gdn_gate_proj(Pj["x"], Pj["W_a"], Pj["W_b"], a=Pj["a"], b=Pj["b"],
                              workspace=Pj["gws"])
            if ev:
                ev[1].record()
            gdn.gdn_linear(Pj["y"], Pj["W_out"], y=Pj["out"], workspace=Pj["lws"])
        fns["proj"] = proj_part

    if "dlayer" in want:
        # The layer's decode step for 64 rows (weights shared with the projections).
        dlx = proj_inputs(R_DECODE, outs=(), gate_H=0, seed=2009)["x"]
        dly = decode_inputs(R_DECODE, seed=2010)
        dlayer = []
        for _ in range(ROT):
            dl = {"x": dev(dlx), "state": dev(dly["state"]), "A_log": dev(dly["A_log"]),
                  "dt_bias": dev(dly["dt_bias"]), "conv_w": dev(mxc["conv_w"]),
                  "norm_w": dev(mxc["norm_w"]),
                  "conv_state": torch.zeros((R_DECODE, 3, C_CONV), dtype=torch.float32,
                                            device="cuda")}
            dl["qkvz"] = torch.empty((R_DECODE, C_CONV + HV * D), dtype=torch.bfloat16,
                                     device="cuda")
            dl["qkv"] = dl["qkvz"][:, :C_CONV].unsqueeze(1)      # [R, 1, 10240], in place
            dl["z"] = dl["qkvz"][:, C_CONV:].unflatten(1, (HV, D))  # [R, 48, 128], in place
            dl["a"] = torch.empty((R_DECODE, HV), dtype=torch.float32, device="cuda")
            dl["b"] = torch.empty((R_DECODE, HV), dtype=torch.float32, device="cuda")
            dl["y"] = torch.empty((R_DECODE, 1, C_CONV), dtype=torch.bfloat16, device="cuda")
            dl["o"] = torch.empty((R_DECODE, HV, D), dtype=torch.bfloat16, device="cuda")
            dl["o2"] = torch.empty((R_DECODE, HV, D), dtype=torch.bfloat16, device="cuda")
            dl["out"] = torch.empty((R_DECODE, HIDDEN), dtype=torch.bfloat16, device="cuda")
            dl["gws"] = torch.empty(
                max(gdn.gdn_gate_proj_workspace_bytes(R_DECODE, HIDDEN, HV), 256),
                dtype=torch.uint8, device="cuda")
            dlayer.append(dl)

        def dlayer_part(i, events=True):
            L = dlayer[i % ROT]
            W = proj[i % ROT]
            ev = dl_ev.get(i) if events else None
            mark = (lambda j: ev[j].record()) if ev else (lambda j: None)
            gdn.gdn_linear(L["x"], W["W_qkvz"], y=L["qkvz"], workspace=W["lws"])
            mark(0)
            gdn.gdn_gate_proj(L["x"], W["W_a"], W["W_b"], a=L["a"], b=L["b"],
                              workspace=L["gws"])
            mark(1)
            gdn.gdn_conv_silu(L["qkv"], L["conv_w"], L["conv_state"], l2_channels=2 * HK * D,
                              y=L["y"])
            mark(2)
            y = L["y"][:, 0]
            gdn.gdn_decode_rows(y[:, :HK * D].unflatten(1, (HK, D)),
                                y[:, HK * D:2 * HK * D].unflatten(1, (HK, D)),
                                y[:, 2 * HK * D:].unflatten(1, (HV, D)), L["a"], L["b"],
                                L["A_log"], L["dt_bias"], L["state"], o=L["o"])
            mark(3)
            gdn.gdn_gated_rmsnorm(L["o"], L["z"], L["norm_w"], y=L["o2"])
            mark(4)
            gdn.gdn_linear(L["o2"].view(R_DECODE, HV * D), W["W_out"], y=L["out"],
                           workspace=W["lws"])
        fns["dlayer"] = dlayer_part

    order = [p for p in PARTS if p in fns]
    log(f"warm-up: {args.warmup} calls of each part: {','.join(order)}")
    for p in order:
        for i in range(args.warmup):
            fns[p](i)
    torch.cuda.synchronize()

    # Each projection shape's plan is timed once here, on a warm GPU and outside
    # the timed loops (gdn_linear alone takes the heuristic's first algorithm
    # that fits), then the parts that use them are warmed up again.
    if "proj" in want or "dlayer" in want:
        Pj = proj[0]
        gdn.gdn_linear_tune(Pj["x"], Pj["W_qkvz"], y=Pj["yin"], workspace=Pj["lws"])
        gdn.gdn_linear_tune(Pj["y"], Pj["W_out"], y=Pj["out"], workspace=Pj["lws"])
    if "dlayer" in want:
        L, W = dlayer[0], proj[0]
        gdn.gdn_linear_tune(L["x"], W["W_qkvz"], y=L["qkvz"], workspace=W["lws"])
        gdn.gdn_linear_tune(L["o2"].view(R_DECODE, HV * D), W["W_out"], y=L["out"],
                            workspace=W["lws"])
    for p in ("proj", "dlayer"):
        if p in fns:
            for i in range(args.warmup):
                fns[p](i)
    torch.cuda.synchronize()

    # The decode step of each buffer set captured in a graph (the plans of its
    # projections were made above, outside the capture).  A
    # capture that fails leaves the part out (graph_us is then null); the
    # replays' results are checked against the eager step in the GPU tests.
    graphs = []
    if "dgraph" in want:
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
            print(f"bench.py: graph capture of the decode step failed ({e}); dgraph skipped",
                  file=sys.stderr)
            graphs = []
            torch.cuda.synchronize()
        if graphs:
            def dgraph_part(i):
                graphs[i % ROT].replay()
            fns["dgraph"] = dgraph_part
            order.append("dgraph")
            for i in range(max(args.warmup, 2)):
                dgraph_part(i)
            torch.cuda.synchronize()

    evs = {p: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for p in order}
    for i in range(args.steps):
        proj_ev[args.warmup + i] = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        dl_ev[args.warmup + i] = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    # The timed region: each part's K calls back to back between one pair of
    # events on the library's stream; the mean per call is what the rates
    # below use.  A second pass with events around every call gives each
    # part's per-call median / min / p90 (an event pair per call adds its own
    # few microseconds) and the split of the multi-call parts.
    reg = {p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for p in order}
    torch.cuda.synchronize()
    log(f"timed: {args.steps} steps")
    t_start = time.perf_counter()
    for p in order:
        reg[p][0].record()
        for i in range(args.steps):
            fns[p](args.warmup + args.steps + i)  # (no per-call events at these indices)
        reg[p][1].record()
        torch.cuda.synchronize()
        log(f"part {p} done")
    wall = time.perf_counter() - t_start
    med = {p: reg[p][0].elapsed_time(reg[p][1]) / args.steps for p in order}  # ms per call

    for p in order:
        for i in range(args.steps):
            evs[p][i][0].record()
            fns[p](args.warmup + i)
            evs[p][i][1].record()
        torch.cuda.synchronize()
    log("per-call pass done")
    per = {p: [evs[p][i][0].elapsed_time(evs[p][i][1]) for i in range(args.steps)]
           for p in order}  # ms per call
    ms_per_step = wall * 1e3 / args.steps

    out = {
        "metric": "GDN layer prefill tokens/s (T=4096) + decode_rows state GB/s at 64 rows",
        "value": round(T_PREFILL / (med["prefill"] * 1e-3), 1) if "prefill" in med else None,
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
                   "value_is": "tokens/s of one gdn_prefill call (the chunked gated delta rule "
                               "alone: chunk_prep + chunk_chain) on the B=1 T=4096 prefill "
                               "workload, mean over the timed calls run back to back; the "
                               "whole mixer at the same size (conv + rule + gated norm) is "
                               "layer_prefill",
                   "step": "one call of each part: " + ", ".join(order)},
    }
    parts_out = {p: dict(region_mean_us=round(med[p] * 1e3, 2), **stats(per[p])) for p in order}
    out["parts_us"] = parts_out
    roofs = {}

    if "prefill" in med:
        t_pre = med["prefill"]
        pre_flops = prefill_flops_per_launch()
        ach_p = pre_flops / (t_pre * 1e-3) / 1e12
        roofs["prefill_b1_t4096"] = {
            "bound": "mfma",
            "kernel": "gdn_prefill chunked: chunk_prep_kernel + chunk_chain_kernel (two launches)",
            "achieved": round(ach_p, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach_p / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": _traffic("prefill_chunked",
                                ["chunk_prefill.hip", "chunk_common.hpp", "common.hpp"]),
            "flops_per_launch": pre_flops, "avg_launch_us": round(t_pre * 1e3, 2),
            "hbm_gbps_algorithmic": round(prefill_bytes_per_launch() / (t_pre * 1e-3) / 1e9, 1)}
    if "decode" in med:
        t_dec = med["decode"]
        dec_bytes = decode_bytes_per_launch()
        state_bytes = 2 * R_DECODE * HV * D * D * 4
        ach_d = dec_bytes / (t_dec * 1e-3) / 1e9
        roofs["decode_rows_r64"] = {
            "bound": "hbm", "kernel": "decode_rows_kernel<bf16,bf16>",
            "achieved": round(ach_d, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach_d / HBM_PEAK_GBPS, 4),
            "traffic": _traffic("decode_rows", ["recurrent.hip", "common.hpp"]),
            "bytes_per_launch": dec_bytes, "avg_launch_us": round(t_dec * 1e3, 2)}
        out["decode_rows"] = {"value": round(state_bytes / (t_dec * 1e-3) / 1e9, 1),
                              "unit": "GB/s (state bytes read+written)",
                              "workload": "decode_rows_r64", "call_us": round(t_dec * 1e3, 2),
                              "frac_of_hbm_peak": round(state_bytes / (t_dec * 1e-3) / 1e9
                                                        / HBM_PEAK_GBPS, 4)}
    if "layer" in med:
        t_layer = med["layer"]
        out["layer_prefill"] = {"value": round(T_PREFILL / (t_layer * 1e-3), 1),
                                "unit": "tokens/s",
                                "workload": "gdn_mixer_prefill (conv+silu+L2 -> chunked prefill "
                                            "-> gated RMSNorm), B=1 T=4096, 10240 conv channels, "
                                            "qkv and z read in place from one [4096, 16384] "
                                            "buffer",
                                "call_us": round(t_layer * 1e3, 2)}
    if "mixer_b4" in med:
        t3 = med["mixer_b4"]
        fused, unfused = mixer_bytes(B3, T3)
        flops3 = prefill_flops_per_launch(T=T3) * B3
        ach3 = fused / (t3 * 1e-3) / 1e9
        out["mixer_b4_t8192"] = {
            "value": round(B3 * T3 / (t3 * 1e-3), 1), "unit": "tokens/s",
            "workload": "mixer_bf16_b4_t8192: one gdn_mixer_prefill call, B=4, T=8192, bf16, "
                        "zero initial states", "call_us": round(t3 * 1e3, 2),
            "mfma_tflops_chunked_form": round(flops3 / (t3 * 1e-3) / 1e12, 2)}
        roofs["mixer_b4_t8192"] = {
            "bound": "hbm", "kernel": "gdn_mixer_prefill (conv, chunk_prep, chunk_chain, norm)",
            "achieved": round(ach3, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach3 / HBM_PEAK_GBPS, 4),
            "traffic": _traffic("mixer_b4_t8192", MIXER_SRC),
            "bytes_per_launch": fused, "bytes_note": "fused minimum (qkv, z, a, b in; y and "
                                                     "state out)",
            "unfused_bytes": unfused,
            "frac_of_unfused_roof": round(unfused / (t3 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "avg_launch_us": round(t3 * 1e3, 2)}
    if "long" in med:
        t4 = med["long"]
        flops4 = prefill_flops_per_launch() * N4
        ach4 = flops4 / (t4 * 1e-3) / 1e12
        out["long_prefill_t65536"] = {
            "value": round(T4 / (t4 * 1e-3), 1), "unit": "tokens/s",
            "workload": "prefill_bf16_b1_t65536_x16: 16 gdn_prefill calls of 4096 tokens, the "
                        "f32 state handed between them", "us": round(t4 * 1e3, 2)}
        roofs["long_prefill_t65536_x16"] = {
            "bound": "mfma", "kernel": "16 x gdn_prefill chunked (chunk_prep + chunk_chain)",
            "achieved": round(ach4, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach4 / BF16_MFMA_PEAK_TFLOPS, 4),
            # the same two kernels as the prefill part, once per 4096-token call
            "traffic": (lambda t: t * N4 if t else None)(
                _traffic("prefill_chunked", ["chunk_prefill.hip", "chunk_common.hpp",
                                             "common.hpp"])),
            "flops": flops4, "us": round(t4 * 1e3, 2),
            "hbm_gbps_algorithmic": round(prefill_bytes_per_launch() * N4 / (t4 * 1e-3) / 1e9,
                                          1)}
    if "slots" in med:
        t_slots = med["slots"]
        out["prefill_slots"] = {
            "value": round(slot_tokens / (t_slots * 1e-3), 1), "unit": "tokens/s",
            "workload": "prefill_slots_bf16_r16 (16 fixed rows, U{1..1024} new tokens each, "
                        "%d tokens, longest %d)" % (slot_tokens, sx["max_len"]),
            "call_us": round(t_slots * 1e3, 2),
            "mfma_tflops": round(slots_flops(sx) / (t_slots * 1e-3) / 1e12, 2)}
    if "multi" in med:
        t_multi = med["multi"]
        multi_bytes = (2 + 4) * R_DECODE * HV * D * D * 4  # state in + out, 4 snapshots
        out["decode_rows_multi"] = {
            "value": round(4 * R_DECODE / (t_multi * 1e-3), 1), "unit": "tokens/s",
            "workload": "decode_rows_r64_k4 (64 rows x 4 draft tokens, state snapshot after "
                        "every token)", "call_us": round(t_multi * 1e3, 2),
            "state_gbps": round(multi_bytes / (t_multi * 1e-3) / 1e9, 1)}
    if "proj" in med:
        t_proj = med["proj"]
        pc = np.median(np.array(
            [[evs["proj"][i][0].elapsed_time(proj_ev[args.warmup + i][0]),
              proj_ev[args.warmup + i][0].elapsed_time(proj_ev[args.warmup + i][1]),
              proj_ev[args.warmup + i][1].elapsed_time(evs["proj"][i][1])]
             for i in range(args.steps)]), axis=0)  # ms
        t_qkvz, t_gate, t_out = pc
        gemm_flops = (2.0 * T_PREFILL * HIDDEN * (C_CONV + HV * D)
                      + 2.0 * T_PREFILL * HV * D * HIDDEN)
        gemm_tflops = gemm_flops / ((t_qkvz + t_out) * 1e-3) / 1e12
        gate_bytes = T_PREFILL * HIDDEN * 2 + 2 * HV * HIDDEN * 4 + 2 * T_PREFILL * HV * 4
        out["projections"] = {
            "workload": "in_proj_qkv 5120->10240 and in_proj_z 5120->6144 as one product "
                        "with the stacked [16384, 5120] weight (bf16, gdn_linear), in_proj_a/b "
                        "5120->48 (f32 weights, gdn_gate_proj), out_proj 6144->5120 (bf16, "
                        "gdn_linear) at 4096 tokens",
            "call_us": round(t_proj * 1e3, 2),
            "in_proj_qkvz_us": round(t_qkvz * 1e3, 2),
            "gate_proj_us": round(t_gate * 1e3, 2), "out_proj_us": round(t_out * 1e3, 2),
            "gemm_tflops": round(gemm_tflops, 1),
            "gemm_frac_of_bf16_peak": round(gemm_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "gate_proj_gbps_algorithmic": round(gate_bytes / (t_gate * 1e-3) / 1e9, 1)}
        if "layer" in med:
            out["full_layer_prefill"] = {
                "value": round(T_PREFILL / ((med["layer"] + t_proj) * 1e-3), 1),
                "unit": "tokens/s",
                "workload": "projections + gdn_mixer_prefill at B=1 T=4096, the two parts' "
                            "mean times added",
                "us": round((med["layer"] + t_proj) * 1e3, 2)}
    if "dlayer" in med:
        t_dl = med["dlayer"]
        t_dg = med.get("dgraph")
        dlc = np.median(np.array(
            [[e[j].elapsed_time(e[j + 1]) for j in range(6)]
             for e in ([evs["dlayer"][i][0]] + dl_ev[args.warmup + i] + [evs["dlayer"][i][1]]
                       for i in range(args.steps))]), axis=0)  # ms
        out["full_layer_decode"] = {
            "value": round(R_DECODE / (t_dl * 1e-3), 1), "unit": "tokens/s",
            "workload": "one decode step of the whole layer for 64 fixed rows: in_proj_qkvz "
                        "(one product), gate projections, conv over one token with the rows' "
                        "conv history, decode_rows, gated RMSNorm, out_proj",
            "us": round(t_dl * 1e3, 2),
            "graph_us": round(t_dg * 1e3, 2) if t_dg else None,
            "graph_value": round(R_DECODE / (t_dg * 1e-3), 1) if t_dg else None,
            "calls_us": dict(zip(["in_proj_qkvz", "gate_proj", "conv",
                                  "decode_rows", "gated_rmsnorm", "out_proj"],
                                 [round(v * 1e3, 2) for v in dlc]))}

    # The dominant kernel of the step: the chunked prefill's two launches (they
    # also carry the long prefill, the ragged batch and the whole mixer's
    # recurrence); decode_rows and the whole mixer in roofline_other.
    if "prefill_b1_t4096" in roofs:
        out["roofline"] = roofs.pop("prefill_b1_t4096")
    elif roofs:
        out["roofline"] = roofs.pop(next(iter(roofs)))
    out["roofline_other"] = roofs

    if not args.no_copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for i in range(5):
            ce[i].record()
            dst.copy_(src)
        ce[5].record()
        torch.cuda.synchronize()
        ts = [ce[i].elapsed_time(ce[i + 1]) for i in range(1, 5)]
        out["copy_256MiB"] = {"GBps": round(2 * src.numel() * 4 / (float(np.median(ts)) * 1e-3)
                                            / 1e9, 1),
                              "note": "device-to-device copy of 256 MiB (read + write bytes), "
                                      "median of 4 after one warm-up"}
        del src, dst
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline and "prefill" in want:
        log("cpu baseline (f64 oracle)")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
