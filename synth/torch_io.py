"""Moving the seeded numpy inputs to and from the GPU with torch (bf16 arrays
travel as their 16-bit patterns).  Plumbing only."""
import numpy as np

from .inputs import to_f64


def dev(a, device="cuda"):
    """numpy (f32, int32, or uint16 bf16 bits) -> torch tensor on the GPU."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host_f64(t):
    """GPU tensor -> exact f64 numpy array."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)
