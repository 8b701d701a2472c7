"""Shared helpers of the GPU tests (no method arithmetic here)."""
import numpy as np
import torch


def rel_err(got, ref):
    """max |got - ref| / rms(ref), over all elements."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.abs(got - ref).max() / max(rms, 1e-300))


def np64(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu")
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def randn(shape, seed, scale=1.0, shift=0.0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * scale + shift
    return x.to(dtype)


def banner(msg):
    print("[case] " + msg, flush=True)
