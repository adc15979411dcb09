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


def chunk_step_bwd(S, X, dO, q, k, v, g, beta):
    """Gradients through one chunk, restated from the chunk form above by reverse mode.

    S: chunk-start state [K,V]; X: gradient with respect to the chunk-end state S';
    dO: gradient with respect to the chunk's outputs [n,V]. Returns the gradient with respect
    to S and (dq, dk, dv, dg, dbeta) of the chunk's tokens. With Qe = Q e^b, Ke = K e^b,
    Kn = K e^{-b}, Kt = K e^{b_last - b} and gamma = e^{b_last}:
      dDelta = P^T dO + Kt X,        dS = Qe^T dO + Diag(gamma) X - W^T dDelta
      dQe = dO S^T + dP Kn,          dP = lower_incl(dO Delta^T)
      dKt = Delta X^T,               dgamma = rowsum(S * X)
      dU = dDelta, dW = -dDelta S^T, dV = diag(beta) T^T dU
      dT = dU (beta V)^T + dW (beta Ke)^T,   dA = strict_lower(-T^T dT T^T)
      dKe = diag(beta) (T^T dW + dA Kn),      dKn = dA^T diag(beta) Ke + dP^T Qe
      dbeta = rowsum(V * T^T dU) + rowsum(Ke * T^T dW) + rowsum(dA * Ke Kn^T)
      db = dQe*Qe + dKe*Ke - dKn*Kn - dKt*Kt, plus sum_i dKt_i*Kt_i + dgamma*gamma on the last
      token; dg_s = sum_{i >= s} db_i, dq = dQe e^b, dk = dKe e^b + dKn e^{-b} + dKt e^{b_last-b}.
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    n = q.shape[0]
    b = np.cumsum(g, axis=0)
    eb, enb = np.exp(b), np.exp(-b)
    gam = np.exp(b[-1])
    Qe, Ke, Kn = q * eb, k * eb, k * enb
    Kt = k * np.exp(b[-1][None, :] - b)
    lower = np.tril(np.ones((n, n)), -1)
    lower_incl = np.tril(np.ones((n, n)), 0)
    KK = Ke @ Kn.T
    A = beta[:, None] * KK * lower
    P = (Qe @ Kn.T) * lower_incl
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ (beta[:, None] * Ke)
    U = T @ (beta[:, None] * v)
    Delta = U - W @ S
    dDelta = P.T @ dO + Kt @ X
    dS = Qe.T @ dO + gam[:, None] * X - W.T @ dDelta
    dP = (dO @ Delta.T) * lower_incl
    dQe = dO @ S.T + dP @ Kn
    dKt = Delta @ X.T
    dgam = np.sum(S * X, axis=1)
    dU, dW = dDelta, -dDelta @ S.T
    TtdU, TtdW = T.T @ dU, T.T @ dW
    dv = beta[:, None] * TtdU
    dT = dU @ (beta[:, None] * v).T + dW @ (beta[:, None] * Ke).T
    dA = (-T.T @ dT @ T.T) * lower
    dKe = beta[:, None] * (TtdW + dA @ Kn)
    dKn = dA.T @ (beta[:, None] * Ke) + dP.T @ Qe
    dbeta = np.sum(v * TtdU, axis=1) + np.sum(Ke * TtdW, axis=1) + np.sum(dA * KK, axis=1)
    db = dQe * Qe + dKe * Ke - dKn * Kn - dKt * Kt
    db[-1] += np.sum(dKt * Kt, axis=0) + dgam * gam
    dg = np.cumsum(db[::-1], axis=0)[::-1]
    dq = dQe * eb
    dk = dKe * eb + dKn * enb + dKt * np.exp(b[-1][None, :] - b)
    return dS, dq, dk, dv, dg, dbeta


def chunk_bwd(q, k, v, g, beta, dO, C, dfinal=None, cu_seqlens=None, init_state=None):
    """Chunkwise gradients over packed sequences: chunk-start states from a forward pass,
    then the chunks in reverse with the running state gradient."""
    q = np.asarray(q, np.float64)
    T, H, K = q.shape
    V = np.asarray(v).shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    dq, dk, dg = (np.zeros((T, H, K)) for _ in range(3))
    dv = np.zeros((T, H, V))
    dbeta = np.zeros((T, H))
    dinit = np.zeros((N, H, K, V))
    for n in range(N):
        for h in range(H):
            S = np.zeros((K, V)) if init_state is None else np.array(init_state[n, h], np.float64)
            starts = list(range(int(cu[n]), int(cu[n + 1]), C))
            states = []
            for s in starts:
                e = min(s + C, int(cu[n + 1]))
                states.append(S)
                _, S = chunk_step(S, q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h], beta[s:e, h])
            X = np.zeros((K, V)) if dfinal is None else np.array(dfinal[n, h], np.float64)
            for s, S0 in zip(starts[::-1], states[::-1]):
                e = min(s + C, int(cu[n + 1]))
                X, a, b_, c, d, f = chunk_step_bwd(S0, X, dO[s:e, h], q[s:e, h], k[s:e, h], v[s:e, h],
                                                   g[s:e, h], beta[s:e, h])
                dq[s:e, h], dk[s:e, h], dv[s:e, h], dg[s:e, h], dbeta[s:e, h] = a, b_, c, d, f
            dinit[n, h] = X
    return dq, dk, dv, dg, dbeta, dinit
