"""Shared test helpers: numpy <-> torch for the stored tensor formats, and the
relative Frobenius metric."""
import numpy as np

import oracle


def to_dev(x, device="cuda"):
    """numpy array in a storage format (bf16 bits as uint16, fp16, fp32,
    int32) -> torch device tensor of the matching dtype."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_np(t):
    """torch tensor -> numpy float64 (bf16 widened exactly)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(
            np.float32).astype(np.float64)
    return t.to(torch.float64).numpy()


rel_fro = oracle.rel_fro
