"""KDA oracle-C: an independent fp64 numpy evaluation of the chunkwise form.

TEST INFRASTRUCTURE ONLY. The product path never imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares
no code with the HIP kernels.

This is the chunkwise algorithm of "Kimi Linear: An Expressive, Efficient
Attention Architecture" (paper-graph-ui review), section "Chunkwise
Parallelization", written out step by step in fp64 for small inputs:

* chunks of C tokens that never cross a sequence boundary;
* g_r = sum_{j<=r} log(alpha_j) inside the chunk (Gamma^{1->C} has rows
  exp(g_r)); the relative decay from token i to token r is exp(g_r - g_i);
* the WY auxiliaries w_r, u_r (review, "The WY representation for P and H")
  and, independently, their UT-transform form
  M = (I + StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T))^{-1} Diag(beta),
  W = M (Gamma*K), U = M V, with the unit-lower-triangular inverse taken by
  forward substitution ("The UT transform for hardware efficiency");
* the chunk state update S' = Diag(gamma_C) S + (Gamma^{i->C}*K)^T (U - W S)
  (Eq. 8, "Chunk-level state update");
* the chunk output O = (Gamma*Q) S + Tril((Gamma*Q)(K/Gamma)^T)(U - W S)
  (Eq. 9, "Output computation").

Following the review's "Numerical stability via secondary chunking", no 1/Gamma
is ever formed: every decayed inner product uses exp(g_r - g_i) per pair.

Reading of a garbled point: the review defines the decay from i to r as a
product over j = i..r, which includes alpha_i. The recurrence (Eq. 1) and the
matrix forms built on Gamma^{1->C} both need the product over j = i+1..r,
i.e. exp(g_r - g_i); this module follows the recurrence.
"""
from __future__ import annotations

import numpy as np


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def forward_substitution_inverse(T: np.ndarray) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix, row by row.

    Row r of X = T^{-1} satisfies X[r] = e_r - sum_{i<r} T[r, i] X[i]
    (forward substitution, as the review prescribes instead of a general
    inverse).
    """
    n = T.shape[0]
    X = np.zeros_like(T)
    for r in range(n):
        X[r] = -(T[r, :r] @ X[:r])
        X[r, r] += 1.0
    return X


def decayed_inner_products(A_rows: np.ndarray, B_rows: np.ndarray,
                           g: np.ndarray, inclusive: bool) -> np.ndarray:
    """M[r, i] = sum_c A_rows[r, c] B_rows[i, c] exp(g[r, c] - g[i, c]).

    Kept for i < r (strict) or i <= r (inclusive); zero above. The exponent
    is only evaluated where it is <= 0, so nothing overflows.
    """
    n = g.shape[0]
    r_idx = np.arange(n)[:, None]
    i_idx = np.arange(n)[None, :]
    keep = (i_idx <= r_idx) if inclusive else (i_idx < r_idx)
    diff = g[:, None, :] - g[None, :, :]                    # [r, i, c]
    diff = np.where(keep[:, :, None], diff, -np.inf)
    return np.einsum("rc,ic,ric->ri", A_rows, B_rows, np.exp(diff))


def wy_auxiliaries(K, V, beta, g):
    """w_r and u_r by the WY recursions of the review (Propositions 1-2).

    w_r = beta_r (Diag(gamma_r) k_r - sum_{i<r} w_i (k_i^T Diag(gamma_{i->r}) k_r))
    u_r = beta_r (v_r - sum_{i<r} u_i (k_i^T Diag(gamma_{i->r}) k_r))
    with gamma_r = exp(g_r) and gamma_{i->r} = exp(g_r - g_i).
    """
    n = K.shape[0]
    w = np.zeros_like(K)
    u = np.zeros_like(V)
    for r in range(n):
        acc_w = np.exp(g[r]) * K[r]
        acc_u = V[r].copy()
        for i in range(r):
            s = np.sum(K[i] * np.exp(g[r] - g[i]) * K[r])
            acc_w = acc_w - w[i] * s
            acc_u = acc_u - u[i] * s
        w[r] = beta[r] * acc_w
        u[r] = beta[r] * acc_u
    return w, u


def chunk_step(S, Q, K, V, la, b):
    """One chunk of the chunkwise algorithm. Returns (O, S_next, parts)."""
    g = np.cumsum(la, axis=0)                      # g_r, inclusive from chunk start
    Gam = np.exp(g)                                # rows of Gamma^{1->C}
    Akk = decayed_inner_products(K, K, g, inclusive=False)
    Aqk = decayed_inner_products(Q, K, g, inclusive=True)
    L = b[:, None] * Akk                           # StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T)
    Ti = forward_substitution_inverse(np.eye(len(b)) + L)
    W = Ti @ (b[:, None] * (Gam * K))              # W = M (Gamma*K), M = Ti Diag(beta)
    U = Ti @ (b[:, None] * V)                      # U = M V
    Vp = U - W @ S                                 # pseudo-value
    O = (Gam * Q) @ S + Aqk @ Vp                   # Eq. 9
    gC = g[-1]
    S_next = np.exp(gC)[:, None] * S + (K * np.exp(gC[None, :] - g)).T @ Vp   # Eq. 8
    parts = dict(g=g, Akk=Akk, L=L, Ti=Ti, W=W, U=U, Aqk=Aqk, S0=S.copy(), Vp=Vp)
    return O, S_next, parts


def chunk_forward(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None,
                  chunk: int = 64, keep_parts: bool = False):
    """fp64 chunkwise KDA forward over packed sequences.

    Shapes: q, k [T, H, dk]; v [T, H, dv]; log_alpha [T, H, dk];
    beta [T, H]; h0 [N, H, dk, dv] or None; cu_seqlens [N+1] or None (one
    sequence). Returns (o [T, H, dv], h_final [N, H, dk, dv], parts) where
    parts[(n, h)] is the list of per-chunk intermediates when keep_parts.
    """
    q, k, v, log_alpha, beta = map(_as64, (q, k, v, log_alpha, beta))
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    h0 = np.zeros((N, H, dk, dv)) if h0 is None else _as64(h0)
    o = np.zeros((T, H, dv))
    h_final = np.zeros((N, H, dk, dv))
    parts = {}
    for n in range(N):
        for h in range(H):
            S = h0[n, h].copy()
            plist = []
            for s in range(cu[n], cu[n + 1], chunk):
                e = min(s + chunk, cu[n + 1])
                O, S, p = chunk_step(S, q[s:e, h], k[s:e, h], v[s:e, h],
                                     log_alpha[s:e, h], beta[s:e, h])
                o[s:e, h] = O
                if keep_parts:
                    p["start"] = s
                    plist.append(p)
            h_final[n, h] = S
            if keep_parts:
                parts[(n, h)] = plist
    return o, h_final, parts
