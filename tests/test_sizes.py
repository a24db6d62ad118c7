"""The workload dimensions reproduce the sizes the pages print
(tests/golden/sizes.json, each item with its source)."""
import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sizes.json")


def _derived():
    d, hk, hv, w = synth.D, synth.HK, synth.HV, synth.CONV_W
    C = synth.CONV_CH
    hidden = 5120  # model width (llm-arch-viz dimensions: hidden 5,120)
    mixer_params = (C * hidden          # in_proj_qkv
                    + hv * d * hidden   # in_proj_z
                    + 2 * hv * hidden   # in_proj_a, in_proj_b
                    + hidden * hv * d   # out_proj
                    + C * w             # conv1d, no bias
                    + d                 # gated norm weight
                    + 2 * hv)           # A_log, dt_bias
    return {
        "conv channels": C,
        "conv width": w,
        "conv1d parameters (no bias)": C * w,
        "gated norm weight width": d,
        "in_proj_z output width": hv * d,
        "per-head parameter vectors (A_log, dt_bias)": hv,
        "GDN mixer parameters": mixer_params,
        "fixed GDN state of the 48 linear layers, bytes at f32, one row": 48 * hv * d * d * 4,
        "norm epsilon": 1e-6,
    }


def test_sizes_match_pages():
    g = json.load(open(GOLDEN))
    got = _derived()
    for item in g["items"]:
        v = got[item["name"]]
        if "value" in item:
            assert v == item["value"], item
        else:
            assert abs(v - item["value_approx"]) <= item["tolerance"], (item, v)
    assert synth.CONV_CH == 2 * synth.HK * synth.D + synth.HV * synth.D
