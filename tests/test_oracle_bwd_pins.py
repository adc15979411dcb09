"""Pins of the oracle's gradients (kda_bwd) against facts independent of its code: central
finite differences of the forward oracle in fp64, and closed forms at beta = 0."""
import numpy as np
import pytest

import oracle


def _inputs(rng, T, H, K, V, N=1):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K)) / np.sqrt(K)
    v = rng.standard_normal((T, H, V))
    g = np.log(rng.uniform(0.4, 1.0, (T, H, K)))
    beta = rng.uniform(0.05, 1.0, (T, H))
    S0 = rng.standard_normal((N, H, K, V))
    return q, k, v, g, beta, S0


def _loss(args, do, dfin, cu):
    q, k, v, g, b, S0 = args
    o, fin = oracle.kda_fwd(q, k, v, g, b, cu_seqlens=cu, init_state=S0)
    return float(np.sum(o * do) + np.sum(fin * dfin))


@pytest.mark.parametrize("lengths,H,K,V", [([7], 2, 3, 4), ([4, 0, 6], 1, 4, 3), ([9], 1, 2, 5)])
def test_gradients_match_central_differences(lengths, H, K, V):
    """Every element of every gradient against (L(x + h) - L(x - h)) / 2h, h = 1e-5."""
    rng = np.random.default_rng(sum(lengths) * 10 + K)
    T, N = sum(lengths), len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    args = list(_inputs(rng, T, H, K, V, N))
    do = rng.standard_normal((T, H, V))
    dfin = rng.standard_normal((N, H, K, V))
    grads = oracle.kda_bwd(*args[:5], do, dfinal=dfin, cu_seqlens=cu, init_state=args[5])
    h = 1e-5
    for which in range(6):
        x = args[which]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(args, do, dfin, cu)
            x[idx] = keep - h
            lm = _loss(args, do, dfin, cu)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(grads[which], fd, rtol=0, atol=1e-7 * scale,
                                   err_msg="gradient %d" % which)


def test_zero_beta_closed_forms():
    """beta = 0 writes nothing: o_t = (prod_{s<=t} Diag(a_s) S0)^T q_t, so dv = 0, dk = 0,
    d S0 = sum_t Diag(prod a) q_t do_t^T + Diag(prod over all a) dfinal, and
    dlog a_{s,c} = sum_{t>=s} q_tc A_tc (S0 do_t)_c + A_Tc (S0 dfinal^T-row sums)_c."""
    rng = np.random.default_rng(3)
    T, K, V = 6, 3, 4
    q, k, v, g, _, S0 = _inputs(rng, T, 1, K, V)
    beta = np.zeros((T, 1))
    do = rng.standard_normal((T, 1, V))
    dfin = rng.standard_normal((1, 1, K, V))
    dq, dk, dv, dg, db, dS0 = oracle.kda_bwd(q, k, v, g, beta, do, dfinal=dfin, init_state=S0)
    assert np.all(dv == 0.0) and np.all(dk == 0.0)
    A = np.exp(np.cumsum(g[:, 0, :], axis=0))  # [T, K] cumulative decay
    ref = sum(np.outer(A[t] * q[t, 0], do[t, 0]) for t in range(T)) + A[-1][:, None] * dfin[0, 0]
    np.testing.assert_allclose(dS0[0, 0], ref, rtol=1e-12, atol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(dq[t, 0], (A[t][:, None] * S0[0, 0]) @ do[t, 0], rtol=1e-12, atol=1e-12)
    # dL/dg_s = sum over t >= s of the terms that contain A_t
    term = np.array([A[t] * q[t, 0] * (S0[0, 0] @ do[t, 0]) for t in range(T)])  # [T, K]
    fin_term = A[-1] * np.sum(S0[0, 0] * dfin[0, 0], axis=1)
    ref_dg = np.cumsum(term[::-1], axis=0)[::-1] + fin_term[None, :]
    np.testing.assert_allclose(dg[:, 0], ref_dg, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("options", [
    oracle.OPT_L2NORM_QK | oracle.OPT_GATE_LOGITS | oracle.OPT_BETA_LOGITS,
    oracle.OPT_SCALAR_GATE | oracle.OPT_GATE_LOGITS,
    oracle.OPT_SCALAR_GATE | oracle.OPT_L2NORM_QK,
])
def test_option_gradients_match_central_differences(options):
    """kda_bwd_options (the chain rule through the input options) against central differences
    of the forward oracle run on apply_options of the raw inputs, for q, k, the gate and beta."""
    rng = np.random.default_rng(options)
    lengths, H, K, V = [5, 0, 4], 1, 3, 2
    T, N = sum(lengths), len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    gshape = (T, H) if options & oracle.OPT_SCALAR_GATE else (T, H, K)
    z = rng.uniform(-2.0, 3.0, gshape) if options & oracle.OPT_GATE_LOGITS else \
        np.log(rng.uniform(0.4, 1.0, gshape))
    b = rng.uniform(-2.0, 2.0, (T, H)) if options & oracle.OPT_BETA_LOGITS else \
        rng.uniform(0.05, 1.0, (T, H))
    S0 = rng.standard_normal((N, H, K, V))
    do = rng.standard_normal((T, H, V))
    dfin = rng.standard_normal((N, H, K, V))
    grads = oracle.kda_bwd_options(q, k, v, z, b, do, options, dfinal=dfin, cu_seqlens=cu,
                                   init_state=S0)
    args = [q, k, v, z, b]

    def loss():
        qp, kp, gp, bp = oracle.apply_options(q, k, z, b, options)
        o, fin = oracle.kda_fwd(qp, kp, v, gp, bp, cu_seqlens=cu, init_state=S0)
        return float(np.sum(o * do) + np.sum(fin * dfin))

    h = 1e-6
    for which in (0, 1, 3, 4):
        x = args[which]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[idx]
            x[idx] = keep + h
            lp = loss()
            x[idx] = keep - h
            lm = loss()
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.abs(fd).max()))
        assert grads[which].shape == x.shape
        np.testing.assert_allclose(grads[which], fd, rtol=0, atol=1e-7 * scale,
                                   err_msg="gradient %d" % which)
