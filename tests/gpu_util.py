"""Moving the seeded numpy inputs to and from the GPU (bf16 arrays travel as
their 16-bit patterns), plus per-test case banners."""
import sys

import numpy as np
import torch

from synth import to_f64


def dev(a, device="cuda"):
    """numpy (f32, int32, or uint16 bf16 bits) -> torch tensor on the GPU."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host_f64(t):
    """GPU tensor -> exact f64 numpy array."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def banner(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)
