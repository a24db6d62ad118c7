"""gdn_prefill_noalloc, the prefill entry point for callers that cannot
allocate device memory (its chunked scratch is a fixed device array of the
library), against gdn_prefill with a caller workspace on the same inputs:
the same kernels and arithmetic, so the same bits; and against the f64
oracle (bar 2e-2 for bf16 inputs, 1e-4 for f32).  Two calls in a row, the
second smaller than the first (the array keeps the first call's contents);
a size beyond the array is refused with nothing enqueued."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_deltanet_mixer_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from synth import recurrence_inputs, to_f64  # noqa: E402
from tests.conftest import max_rel_err  # noqa: E402
from tests.gpu_util import banner, dev, host_f64  # noqa: E402

GDN_ERR_SCRATCH = 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _both(x):
    """(o, state) of gdn_prefill with a workspace and of gdn_prefill_noalloc."""
    B, T, Hk = x["q"].shape[:3]
    Hv = x["v"].shape[2]
    args = [dev(x[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")]
    si = dev(x["state"])
    s1, s2 = torch.empty_like(si), torch.empty_like(si)
    o1 = gdn.gdn_prefill(*args, si, s1)
    o2 = torch.full_like(o1, float("nan"))
    gdn.gdn_prefill_noalloc(*args, si, s2, o=o2)
    torch.cuda.synchronize()
    return (o1, s1), (o2, s2)


def _oracle(x):
    al, be, _ = oracle.gates(to_f64(x["a"]), to_f64(x["b"]), x["A_log"], x["dt_bias"])
    return oracle.recurrence(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), al, be,
                             to_f64(x["state"]))


def test_noalloc_matches_prefill_on_two_calls_in_a_row():
    # 1: the model's heads at 1024 tokens (56 MiB of the 64 MiB scratch)
    banner("noalloc call 1: B=1 T=1024 Hk=16 Hv=48 bf16")
    x = recurrence_inputs(1, 1024, qkv_dt="bf16", gate_dt="f32", seed=501, state_std=0.05)
    (o1, s1), (o2, s2) = _both(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, S_ref = _oracle(x)
    assert max_rel_err(host_f64(o2), o_ref) < 2e-2
    assert max_rel_err(host_f64(s2), S_ref) < 2e-2
    # 2: a smaller call right after (the scratch holds call 1's contents)
    banner("noalloc call 2: B=2 T=130 Hk=2 Hv=6 bf16")
    x = recurrence_inputs(2, 130, Hk=2, Hv=6, qkv_dt="bf16", gate_dt="bf16", seed=502,
                          state_std=0.05)
    (o1, s1), (o2, s2) = _both(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, S_ref = _oracle(x)
    assert max_rel_err(host_f64(o2), o_ref) < 2e-2
    assert max_rel_err(host_f64(s2), S_ref) < 2e-2


def test_noalloc_f32_and_too_large():
    banner("noalloc f32 (no scratch) and a size beyond the scratch")
    x = recurrence_inputs(1, 70, Hk=2, Hv=6, qkv_dt="f32", gate_dt="f32", seed=503,
                          state_std=0.05)
    (o1, s1), (o2, s2) = _both(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, S_ref = _oracle(x)
    assert max_rel_err(host_f64(o2), o_ref) < 1e-4
    # 1153 tokens at 16/48 heads need more than GDN_NOALLOC_SCRATCH_BYTES
    x = recurrence_inputs(1, 1153, qkv_dt="bf16", gate_dt="f32", seed=504, state_std=0.05)
    need = gdn.gdn_prefill_workspace_bytes(1, 1153, 16, 48)
    assert need > (64 << 20)
    args = [dev(x[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")]
    si = dev(x["state"])
    so = torch.full_like(si, 7.0)
    o = torch.full((1, 1153, 48, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_prefill_noalloc(*args, si, so, o=o)
    assert ei.value.status == GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((so == 7.0).all()) and bool((o == 3.0).all())  # nothing was enqueued
