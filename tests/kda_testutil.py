"""Helpers shared by the GPU tests: host arrays to device tensors and the
error measures the tolerances are stated in."""
import numpy as np
import torch


def dev(x, dtype=torch.float32):
    """numpy -> contiguous device tensor (bf16-exact float32 values convert
    exactly to bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def io_dtype(io):
    return torch.bfloat16 if io == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max_err(got, ref):
    """max |got - ref| / max |ref| (the operator's output tolerance measure)."""
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def rel_fro_err(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


# Tolerances: output max-abs error relative to max|o|; state relative
# Frobenius error. fp32 I/O: 1e-4 on o and (unstated on the pages, chosen
# here) 1e-4 on the state; bf16 I/O: 2e-2 on o, 1e-2 on the state.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}
