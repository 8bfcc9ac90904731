"""Python entry to oracle-R, the fp64 token-by-token recurrence (kda_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

The recurrence is Eq. 1 of the pages ("Kimi Linear: An Expressive, Efficient
Attention Architecture", paper-graph-ui review, section "The KDA State Update
Equation"), with the readout o_t = S_t^T q_t on the updated state.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not _build.LIB.exists():
            _build.build()
        lib = ctypes.CDLL(str(_build.LIB))
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.kda_oracle_forward.argtypes = [d, d, d, d, d, d,
                                           ctypes.POINTER(ctypes.c_int64),
                                           i64, i64, i64, i64, d, d, ctypes.c_int]
        lib.kda_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def host_threads() -> int:
    """Cores this process may run on (the oracle's default thread count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, threads=None):
    """Runs the recurrence over packed sequences.

    q, k [T, H, dk]; v [T, H, dv]; log_alpha [T, H, dk]; beta [T, H];
    h0 [N, H, dk, dv] or None (zeros); cu_seqlens [N+1] or None (one
    sequence of length T). Inputs are widened to fp64 (exact for bf16/fp32
    values). Returns (o [T, H, dv], h_final [N, H, dk, dv]) in fp64.
    """
    q, k, v, log_alpha, beta = (np.ascontiguousarray(x, dtype=np.float64)
                                for x in (q, k, v, log_alpha, beta))
    T, H, dk = k.shape
    dv = v.shape[2]
    assert q.shape == (T, H, dk) and log_alpha.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    cu = np.ascontiguousarray([0, T] if cu_seqlens is None else cu_seqlens,
                              dtype=np.int64)
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64)
        assert h0.shape == (N, H, dk, dv)
    o = np.empty((T, H, dv), dtype=np.float64)
    h_final = np.empty((N, H, dk, dv), dtype=np.float64)
    rc = _lib().kda_oracle_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, H, dk, dv,
        _ptr(o), _ptr(h_final), int(threads or host_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return o, h_final


L2NORM_EPS = 1e-6


def l2norm(x, eps=L2NORM_EPS):
    """Scales each vector along the last axis to unit Euclidean length,
    x / sqrt(sum_c x_c^2 + eps), in fp64.

    The pages apply L2Norm to q and k ("Kimi Linear" review, section
    "Neural Parameterization": q and k are normalised to unit length so the
    rank-1 Householder correction stays well behaved; the "L2 Deep Distill"
    page fuses it into the operator). The pages give no epsilon; eps = 1e-6
    keeps a zero vector at zero and changes a unit-scale vector by ~1e-7.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def decode_step(q, k, v, log_alpha, beta, S, threads=None):
    """One recurrent step for N sequences x H heads (one token each).

    q, k, log_alpha [N, H, dk]; v [N, H, dv]; beta [N, H]; S [N, H, dk, dv].
    Returns (o [N, H, dv], S_next [N, H, dk, dv]) in fp64; S is not modified.
    A decode step is the recurrence over N one-token sequences.
    """
    N = np.shape(k)[0]
    return forward(q, k, v, log_alpha, beta, h0=S,
                   cu_seqlens=np.arange(N + 1), threads=threads)
