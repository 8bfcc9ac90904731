"""fp64 oracle of the output epilogue: head-wise RMSNorm times a sigmoid gate.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

The pages put a head-wise RMSNorm and a data-dependent sigmoid gate between
the operator and the output projection ("Kimi Linear" review, section
"Neural Parameterization", output gate equation; the "L2 Deep Distill"
page names the fused form FusedRMSNormGated):
    y = sigmoid(g) * RMSNorm(o),   RMSNorm(o) = o / sqrt(mean_j o_j^2 + eps) * w
per (token, head) over the d_v channels, with g the gate pre-activation of
that head (the low-rank projection's output) and w the norm's per-channel
weight. The pages give neither eps nor the weight's form; the reading here
is one weight vector of d_v entries shared by all heads (None = ones) and
eps passed by the caller.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    """1 / (1 + e^-x) in fp64, written so neither branch overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def rmsnorm_gate(o, g, weight=None, eps=1e-6):
    """o, g [..., d_v]; weight [d_v] or None. Returns y [..., d_v] in fp64."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return sigmoid(g) * y
