"""CPU fp64 chunkwise form of KDA (numpy), a test tool.

It restates, from the token recurrence, the chunkwise algebra that the GPU kernels
implement, so that the algebra itself can be checked against the oracle on the CPU.
It is not the oracle and shares no code with the HIP path.

Chunkwise structure from "Kimi Linear's Hybrid Linear Attention Architecture: A Technical
Breakdown", section 4 "Hardware-Friendly Chunkwise Computation" (state passing with the
cumulative in-chunk decay, the K / U / W matrix forms and the masked intra-chunk output),
and the WY / triangular-solve representation of the chunk's rank-1 updates ("Kimi Linear"
explainer, "WY Representation"; wpnews article, DPLR paragraph). The superscripts printed
on the pages are garbled, so the exact exponents below are derived from the recurrence:

  b_i   = sum_{s<=i} g_s                (per key channel, within the chunk)
  A_ij  = beta_i sum_c k_ic k_jc e^{b_ic - b_jc}     j < i   (strictly lower)
  T     = (I + A)^{-1}
  W     = T diag(beta) (K * e^{b});  U = T diag(beta) V
  Delta = U - W S                    (the per-token delta corrections)
  O     = (Q * e^{b}) S + P Delta,   P_ij = sum_c q_ic k_jc e^{b_ic - b_jc}, j <= i
  S'    = Diag(e^{b_last}) S + (K * e^{b_last - b})^T Delta
"""
from __future__ import annotations

import numpy as np


def chunk_step(S, q, k, v, g, beta):
    """One chunk of n tokens; S [K,V] fp64 chunk-start state. Returns (O [n,V], S')."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    n = q.shape[0]
    b = np.cumsum(g, axis=0)                                  # [n, K]
    pair = np.exp(b[:, None, :] - b[None, :, :])              # [i, j, K], e^{b_i - b_j}
    lower = np.tril(np.ones((n, n)), -1)
    lower_incl = np.tril(np.ones((n, n)), 0)
    A = beta[:, None] * np.einsum("ic,jc,ijc->ij", k, k, pair) * lower
    P = np.einsum("ic,jc,ijc->ij", q, k, pair) * lower_incl
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ (beta[:, None] * (k * np.exp(b)))
    U = T @ (beta[:, None] * v)
    Delta = U - W @ S
    O = (q * np.exp(b)) @ S + P @ Delta
    Snew = np.exp(b[-1])[:, None] * S + (k * np.exp(b[-1][None, :] - b)).T @ Delta
    return O, Snew


def chunk_transition(k, g, beta):
    """The chunk's K x K state transition Diag(e^{b_last}) - (K * e^{b_last - b})^T W."""
    k = np.asarray(k, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    n = k.shape[0]
    b = np.cumsum(g, axis=0)
    pair = np.exp(b[:, None, :] - b[None, :, :])
    A = beta[:, None] * np.einsum("ic,jc,ijc->ij", k, k, pair) * np.tril(np.ones((n, n)), -1)
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ (beta[:, None] * (k * np.exp(b)))
    return np.diag(np.exp(b[-1])) - (k * np.exp(b[-1][None, :] - b)).T @ W


def chunk_fwd(q, k, v, g, beta, C, cu_seqlens=None, init_state=None):
    """Chunkwise forward over packed sequences [T, H, .]; chunks restart at each sequence."""
    q = np.asarray(q, np.float64)
    T, H, K = q.shape
    V = np.asarray(v).shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, V))
    fin = np.zeros((N, H, K, V))
    for n in range(N):
        for h in range(H):
            S = np.zeros((K, V)) if init_state is None else np.array(init_state[n, h], np.float64)
            for s in range(int(cu[n]), int(cu[n + 1]), C):
                e = min(s + C, int(cu[n + 1]))
                O, S = chunk_step(S, q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h], beta[s:e, h])
                o[s:e, h] = O
            fin[n, h] = S
    return o, fin
