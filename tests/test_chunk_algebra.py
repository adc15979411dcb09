"""The chunkwise algebra (tests/chunk_ref.py) against the oracle, on the CPU.

This pins the chunk form the GPU kernels implement to the token recurrence: the chunk
result must not depend on the chunk size (C=1 is the recurrence itself), chunks restart at
sequence starts, and the chunk transition equals the product of the per-token DPLR
transitions with a correction of rank at most min(C, K) ("Kimi Linear" explainer, "The
Woodbury Identity Trick": a product of c diagonal-plus-rank-1 matrices is diagonal plus
rank at most c).
"""
import numpy as np
import pytest

import oracle
from chunk_ref import chunk_fwd, chunk_transition


def _inputs(rng, T, H, K, V, alpha_lo=0.5):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = np.log(rng.uniform(alpha_lo, 1.0, (T, H, K)))
    beta = rng.uniform(0, 1, (T, H))
    return [a.astype(np.float32).astype(np.float64) for a in (q, k, v, g, beta)]


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_form_matches_oracle(C):
    rng = np.random.default_rng(C)
    lens = [70, 1, 33, 64, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    K, V, H = 8, 6, 2
    q, k, v, g, beta = _inputs(rng, int(cu[-1]), H, K, V)
    S0 = rng.standard_normal((len(lens), H, K, V))
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=cu, init_state=S0)
    oc, fc = chunk_fwd(q, k, v, g, beta, C, cu_seqlens=cu, init_state=S0)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(fc, fin, rtol=1e-10, atol=1e-10)


def test_chunk_transition_is_product_of_token_transitions():
    rng = np.random.default_rng(21)
    n, K = 5, 9
    k = rng.standard_normal((n, K))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = np.log(rng.uniform(0.4, 1.0, (n, K)))
    beta = rng.uniform(0, 1, n)
    M = np.eye(K)
    for t in range(n):
        a = np.exp(g[t])
        M = (np.diag(a) - beta[t] * np.outer(k[t], a * k[t])) @ M
    Mc = chunk_transition(k, g, beta)
    np.testing.assert_allclose(Mc, M, rtol=1e-12, atol=1e-12)
    corr = np.diag(np.exp(g.sum(0))) - Mc
    assert np.linalg.matrix_rank(corr, tol=1e-10) <= min(n, K)


def test_chunk_form_with_strong_decay():
    """Strong per-channel decay (alpha down to 0.01) through the exact chunk form."""
    rng = np.random.default_rng(22)
    K, V = 8, 4
    q, k, v, g, beta = _inputs(rng, 50, 1, K, V, alpha_lo=0.01)
    o, fin = oracle.kda_fwd(q, k, v, g, beta)
    oc, fc = chunk_fwd(q, k, v, g, beta, 16)
    np.testing.assert_allclose(oc, o, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(fc, fin, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("C", [1, 5, 16, 64])
def test_chunk_gradients_match_oracle(C):
    """The chunk-form gradients (chunk_ref.chunk_bwd) equal the oracle's token-level reverse
    mode for any chunk size, across ragged sequences with initial and final-state gradients."""
    from chunk_ref import chunk_bwd
    rng = np.random.default_rng(100 + C)
    lens = [40, 1, 17, 0, 64]
    T, H, K, V = sum(lens), 2, 6, 5
    q, k, v, g, beta = _inputs(rng, T, H, K, V)
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = rng.standard_normal((len(lens), H, K, V))
    dO = rng.standard_normal((T, H, V))
    dfin = rng.standard_normal((len(lens), H, K, V))
    ref = oracle.kda_bwd(q, k, v, g, beta, dO, dfinal=dfin, cu_seqlens=cu, init_state=S0)
    got = chunk_bwd(q, k, v, g, beta, dO, C, dfinal=dfin, cu_seqlens=cu, init_state=S0)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dinit"), got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(b).max()), err_msg=name)


def test_group_scan_matches_oracle():
    """The scan over groups of chunks, in fp64: one chunked pass per group from the zero state
    with the values widened to [v | 0] and the initial state [0 | I] gives [B_g | M_g] (the
    group's end state from zero and its K x K transition); S_in(g + 1) = M_g S_in(g) + B_g; a
    second chunked pass from S_in(g) reproduces the token recurrence ("Kimi Linear" explainer,
    "DPLR Chunked Parallel"). Slow decay and short groups keep M_g far from zero, so a wrong
    transition would show."""
    rng = np.random.default_rng(23)
    T, H, K, V, C, Lg = 300, 2, 8, 6, 16, 48   # 7 groups, the last one partial
    q, k, v, g, beta = _inputs(rng, T, H, K, V, alpha_lo=0.98)
    S0 = rng.standard_normal((1, H, K, V))
    o_ref, f_ref = oracle.kda_fwd(q, k, v, g, beta, init_state=S0)
    starts = list(range(0, T, Lg))
    o = np.zeros((T, H, V))
    S_in = S0[0].copy()
    mnorm = []
    for s in starts:
        e = min(s + Lg, T)
        sl = slice(s, e)
        vaug = np.concatenate([v[sl], np.zeros((e - s, H, K))], axis=2)
        init1 = np.concatenate([np.zeros((1, H, K, V)), np.broadcast_to(np.eye(K), (1, H, K, K))],
                               axis=3)
        _, f1 = chunk_fwd(q[sl], k[sl], vaug, g[sl], beta[sl], C, init_state=init1)
        B, M = f1[0, :, :, :V], f1[0, :, :, V:]
        mnorm.append(np.abs(M).max())
        og, fg = chunk_fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], C, init_state=S_in[None])
        o[sl] = og
        S_next = np.einsum("hij,hjv->hiv", M, S_in) + B
        np.testing.assert_allclose(S_next, fg[0], rtol=1e-10, atol=1e-10)
        S_in = S_next
    assert min(mnorm) > 1e-2
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S_in, f_ref[0], rtol=1e-10, atol=1e-10)
