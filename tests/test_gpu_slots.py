"""GPU parity of gdn_prefill_slots: a ragged prefill of fixed rows, each row
continuing from its own state with its own number of new tokens, packed on
one token axis.  Checked per row against the f64 oracle (bar 2e-2, bf16
inputs; 1e-4 for f32 inputs, which run token by token in f32) and bitwise
against a separate gdn_prefill call on that row alone (the same chunk
boundaries, or the same sequential kernel, so the same arithmetic); a row with
no tokens keeps its state bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import make_workload, slots_inputs, to_f64  # noqa: E402
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def run_slots(x):
    st = dev(x["state"])
    o = gdn.gdn_prefill_slots(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]), dev(x["b"]),
                              dev(x["A_log"]), dev(x["dt_bias"]), dev(x["cu_seqlens"]), st,
                              x["max_len"])
    torch.cuda.synchronize()
    return o, st


def run_row_alone(x, r):
    """Row r through gdn_prefill (B=1, T=its length): the reference for bits."""
    c0, c1 = int(x["cu_seqlens"][r]), int(x["cu_seqlens"][r + 1])
    S = dev(x["state"][r:r + 1])
    if c1 == c0:
        return None, S
    o = gdn.gdn_prefill(dev(x["q"][c0:c1])[None], dev(x["k"][c0:c1])[None],
                        dev(x["v"][c0:c1])[None], dev(x["a"][c0:c1])[None],
                        dev(x["b"][c0:c1])[None], dev(x["A_log"]), dev(x["dt_bias"]), S, S,
                        algo="auto")
    torch.cuda.synchronize()
    return o[0], S


def oracle_row(x, r, heads=None):
    c0, c1 = int(x["cu_seqlens"][r]), int(x["cu_seqlens"][r + 1])
    Hv = x["v"].shape[1]
    heads = list(range(Hv)) if heads is None else heads
    grp = Hv // x["q"].shape[1]
    q = np.stack([to_f64(x["q"][c0:c1, h // grp]) for h in heads], axis=1)[None]
    k = np.stack([to_f64(x["k"][c0:c1, h // grp]) for h in heads], axis=1)[None]
    v = to_f64(x["v"][c0:c1, heads])[None]
    al, be, _ = oracle.gates(to_f64(x["a"][c0:c1, heads])[None],
                             to_f64(x["b"][c0:c1, heads])[None], x["A_log"][heads],
                             x["dt_bias"][heads])
    # one q/k head per value head: Hk' = Hv' = len(heads)
    return oracle.recurrence(q, k, v, al, be, to_f64(x["state"][r:r + 1, heads]))


@pytest.mark.parametrize("qkv_dt", ["bf16", "f32"])
def test_prefill_slots_ragged_small(qkv_dt):
    lengths = [0, 1, 63, 64, 65, 150, 300, 7]
    banner(f"prefill_slots {qkv_dt} lengths={lengths} Hk=2 Hv=6")
    x = slots_inputs(lengths, Hk=2, Hv=6, qkv_dt=qkv_dt, seed=61)
    o, st = run_slots(x)
    cu = x["cu_seqlens"]
    for r, L in enumerate(lengths):
        o_row, S_row = run_row_alone(x, r)
        if L == 0:
            assert torch.equal(st[r], dev(x["state"][r])), "an empty row changed its state"
            continue
        assert torch.equal(o[cu[r]:cu[r + 1]], o_row), f"row {r}: o differs from a lone call"
        assert torch.equal(st[r:r + 1], S_row), f"row {r}: state differs from a lone call"
        o_ref, S_ref = oracle_row(x, r)
        assert max_rel_err(host_f64(o[cu[r]:cu[r + 1]]), o_ref[0]) < TOL[qkv_dt], r
        assert max_rel_err(host_f64(st[r]), S_ref[0]) < TOL[qkv_dt], r


def test_prefill_slots_wide_chain_ragged():
    """Enough rows that the chain runs 64-column slices (16 rows x 24 value
    heads x 4 narrow slices > 256), with empty, one-token and chunk-edge rows."""
    lengths = [0, 1, 63, 64, 65, 130, 7, 0, 200, 2, 64, 129, 1, 31, 96, 150]
    banner(f"prefill_slots wide chain lengths={lengths} Hk=4 Hv=24")
    x = slots_inputs(lengths, Hk=4, Hv=24, qkv_dt="bf16", seed=62)
    o, st = run_slots(x)
    cu = x["cu_seqlens"]
    for r, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(st[r], dev(x["state"][r])), "an empty row changed its state"
            continue
        o_ref, S_ref = oracle_row(x, r)
        assert max_rel_err(host_f64(o[cu[r]:cu[r + 1]]), o_ref[0]) < TOL["bf16"], r
        assert max_rel_err(host_f64(st[r]), S_ref[0]) < TOL["bf16"], r


def test_prefill_slots_server_batch_full_width():
    """The benchmarked ragged batch (16 rows of the model's layer, 16 q/k and
    48 value heads, U{1..1024} new tokens each): every row bitwise against its
    lone call, two rows against the oracle on sampled heads."""
    x = make_workload("prefill_slots_bf16_r16")
    lengths = np.diff(x["cu_seqlens"])
    banner(f"prefill_slots_bf16_r16 lengths {lengths.min()}..{lengths.max()}")
    o, st = run_slots(x)
    cu = x["cu_seqlens"]
    for r in range(len(lengths)):
        o_row, S_row = run_row_alone(x, r)
        assert torch.equal(o[cu[r]:cu[r + 1]], o_row), r
        assert torch.equal(st[r:r + 1], S_row), r
    heads = [0, 25, 47]
    for r in (int(np.argmax(lengths)), 3):
        o_ref, S_ref = oracle_row(x, r, heads)
        e_o = max_rel_err(host_f64(o[cu[r]:cu[r + 1], heads]), o_ref[0])
        e_s = max_rel_err(host_f64(st[r, heads]), S_ref[0])
        print(f"row {r} (len {lengths[r]}): o err {e_o:.2e}, state err {e_s:.2e}")
        assert e_o < TOL["bf16"] and e_s < TOL["bf16"]
