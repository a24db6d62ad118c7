"""GPU parity of gdn_decode_rows_multi: K draft tokens per fixed row, each
row's state advanced through them in registers, with the state after every
token written to snapshots.  Checked against the f64 oracle token by token
(o per token, every snapshot and the final state; bar 2e-2 for bf16 inputs,
1e-4 for f32) and bitwise against K successive gdn_decode_rows calls."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import decode_multi_inputs, make_workload, to_f64  # noqa: E402
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def run_multi(x, lengths=None, with_snapshots=True):
    R, K, Hv, d = x["v"].shape
    st = dev(x["state"])
    snap = (torch.full((R, K, Hv, d, d), float("nan"), dtype=torch.float32, device="cuda")
            if with_snapshots else None)
    o = gdn.gdn_decode_rows_multi(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["a"]),
                                  dev(x["b"]), dev(x["A_log"]), dev(x["dt_bias"]), st, snap,
                                  lengths=lengths)
    torch.cuda.synchronize()
    return o, st, snap


def run_successive(x, lengths=None):
    """The same K tokens as K separate gdn_decode_rows calls."""
    R, K = x["v"].shape[:2]
    st = dev(x["state"])
    outs, states = [], []
    for t in range(K):
        outs.append(gdn.gdn_decode_rows(dev(x["q"][:, t]), dev(x["k"][:, t]), dev(x["v"][:, t]),
                                        dev(x["a"][:, t]), dev(x["b"][:, t]), dev(x["A_log"]),
                                        dev(x["dt_bias"]), st, lengths=lengths))
        states.append(st.clone())
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1), st, torch.stack(states, dim=1)


def oracle_rows(x, rows, heads=None):
    """Per row: o [K, H', d] and the state after each token [K, H', d, d]."""
    K = x["v"].shape[1]
    Hv, Hk = x["v"].shape[2], x["q"].shape[2]
    heads = list(range(Hv)) if heads is None else heads
    grp = Hv // Hk
    res = []
    for r in rows:
        q = np.stack([to_f64(x["q"][r, :, h // grp]) for h in heads], axis=1)[None]
        k = np.stack([to_f64(x["k"][r, :, h // grp]) for h in heads], axis=1)[None]
        v = to_f64(x["v"][r][:, heads])[None]
        al, be, _ = oracle.gates(to_f64(x["a"][r][:, heads])[None], to_f64(x["b"][r][:, heads])[None],
                                 x["A_log"][heads], x["dt_bias"][heads])
        S = to_f64(x["state"][r:r + 1, heads])
        o_all, snaps = [], []
        for t in range(K):
            o_t, S = oracle.recurrence(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1],
                                       al[:, t:t + 1], be[:, t:t + 1], S)
            o_all.append(o_t[0, 0])
            snaps.append(S[0])
        res.append((np.stack(o_all), np.stack(snaps)))
    return res


@pytest.mark.parametrize("K", [1, 3, 5])
def test_decode_multi_small(K):
    banner(f"decode_rows_multi R=5 K={K} Hk=2 Hv=6, one idle row")
    R = 5
    x = decode_multi_inputs(R, K, Hk=2, Hv=6, seed=70 + K)
    lengths = dev(np.array([3, -1, 100, 7, 1], dtype=np.int32))
    o, st, snap = run_multi(x, lengths)
    o2, st2, states2 = run_successive(x, lengths)
    assert torch.equal(o, o2) and torch.equal(st, st2)
    active = [0, 2, 3, 4]
    assert torch.equal(snap[active], states2[active])
    # idle row: state untouched, outputs zero, snapshots not written
    assert torch.equal(st[1], dev(x["state"][1]))
    assert torch.count_nonzero(o[1]) == 0
    assert torch.isnan(snap[1]).all()
    for r, (o_ref, s_ref) in zip(active, oracle_rows(x, active)):
        assert max_rel_err(host_f64(o[r]), o_ref) < TOL
        assert max_rel_err(host_f64(snap[r]), s_ref) < TOL
        assert max_rel_err(host_f64(st[r]), s_ref[-1]) < TOL


def test_decode_multi_no_snapshots_f32():
    banner("decode_rows_multi f32 R=3 K=4 without snapshots")
    x = decode_multi_inputs(3, 4, Hk=2, Hv=6, qkv_dt="f32", gate_dt="f32", seed=79)
    o, st, _ = run_multi(x, with_snapshots=False)
    for r, (o_ref, s_ref) in enumerate(oracle_rows(x, range(3))):
        assert max_rel_err(host_f64(o[r]), o_ref) < 1e-4
        assert max_rel_err(host_f64(st[r]), s_ref[-1]) < 1e-4


def test_decode_multi_r64_k4_full():
    """The benchmarked shape (64 rows, 4 draft tokens, full width): bitwise
    against 4 successive decode_rows calls, sampled rows against the oracle."""
    x = make_workload("decode_rows_r64_k4")
    banner("decode_rows_r64_k4 full")
    o, st, snap = run_multi(x)
    o2, st2, states2 = run_successive(x)
    assert torch.equal(o, o2) and torch.equal(st, st2) and torch.equal(snap, states2)
    heads = [0, 31, 47]
    for r, (o_ref, s_ref) in zip((0, 63), oracle_rows(x, (0, 63), heads)):
        assert max_rel_err(host_f64(o[r][:, heads]), o_ref) < TOL
        assert max_rel_err(host_f64(snap[r][:, heads]), s_ref) < TOL
