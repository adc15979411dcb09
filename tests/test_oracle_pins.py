"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, transposed S, erase before decay, read before write, a wrong beta weighting,
state leaking across sequences) fails at least one of them. None of them re-types the
oracle's four steps: they use closed forms, invariants, a hand-worked example, a
different algebraic route (explicit DPLR transition matrices) or limits.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, H, K, V, unit_k=True, alpha_lo=0.5):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = np.log(rng.uniform(alpha_lo, 1.0, (T, H, K)))
    beta = rng.uniform(0.0, 1.0, (T, H))
    f = lambda a: a.astype(np.float32).astype(np.float64)  # what the oracle sees
    return f(q), f(k), f(v), f(g), f(beta)


# ---------------------------------------------------------------- hand-worked example
def test_hand_example():
    """Technical Breakdown 3.3 (order), wpnews code block (orientation), explainer Step 4."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_example_k2v2.json")))
    q = np.array(ex["q"])[:, None, :]
    k = np.array(ex["k"])[:, None, :]
    v = np.array(ex["v"])[:, None, :]
    g = np.log(np.array(ex["alpha"]))[:, None, :]
    b = np.array(ex["beta"])[:, None]
    o, fin = oracle.kda_fwd(q, k, v, g, b)
    np.testing.assert_allclose(o[:, 0, :], np.array(ex["o"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(fin[0, 0], np.array(ex["final_state"]), rtol=1e-7, atol=1e-7)


# ---------------------------------------------------------------- pin 1: brute force
def _dplr_bruteforce(q, k, v, g, beta, S0):
    """S_t = A_t S_{t-1} + beta_t k_t v_t^T with the explicit K x K transition
    A_t = Diag(alpha_t) - beta_t k_t (alpha_t * k_t)^T ('diagonal plus rank-1' form of
    the explainer's DPLR section), o_t = S_t^T q_t."""
    T, K = q.shape
    S = S0.copy()
    outs = []
    for t in range(T):
        a = np.exp(g[t])
        At = np.diag(a) - beta[t] * np.outer(k[t], a * k[t])
        S = At @ S + beta[t] * np.outer(k[t], v[t])
        outs.append(S.T @ q[t])
    return np.array(outs), S


@pytest.mark.parametrize("K,V,T", [(3, 5, 7), (8, 4, 16), (6, 6, 11)])
def test_bruteforce_dplr(K, V, T):
    rng = np.random.default_rng(K * 100 + V * 10 + T)
    q, k, v, g, beta = _rand_inputs(rng, T, 2, K, V, unit_k=False, alpha_lo=0.3)
    S0 = rng.standard_normal((1, 2, K, V))
    o, fin = oracle.kda_fwd(q, k, v, g, beta, init_state=S0)
    for h in range(2):
        ob, Sb = _dplr_bruteforce(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h])
        np.testing.assert_allclose(o[:, h], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], Sb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- pin 2: beta = 0
def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    T, K, V = 20, 8, 5
    q, k, v, g, _ = _rand_inputs(rng, T, 1, K, V)
    beta = np.zeros((T, 1))
    S0 = rng.standard_normal((1, 1, K, V))
    o, fin = oracle.kda_fwd(q, k, v, g, beta, init_state=S0)
    gam = np.exp(np.cumsum(g[:, 0], axis=0))  # gamma_t = prod_{s<=t} alpha_s
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], (gam[t][:, None] * S0[0, 0]).T @ q[t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], gam[-1][:, None] * S0[0, 0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- pin 3: exact recall
def test_unit_key_beta_one_recalls_value():
    """Unit-norm k and beta=1 overwrite the memory along k: k_t^T S_t = v_t^T for any alpha."""
    rng = np.random.default_rng(3)
    T, K, V = 12, 6, 4
    q, _, v, g, _ = _rand_inputs(rng, T, 1, K, V, alpha_lo=0.2)
    # keys with +-1/2 on four random channels: exactly unit norm in binary floating point,
    # mutually non-orthogonal in general
    k = np.zeros((T, 1, K))
    for t in range(T):
        idx = rng.choice(K, 4, replace=False)
        k[t, 0, idx] = rng.choice([-0.5, 0.5], 4)
    beta = np.ones((T, 1))
    S0 = rng.standard_normal((1, 1, K, V))
    # run token by token through the oracle's fwd with state hand-off to see every S_t
    S = S0
    for t in range(T):
        _, S = oracle.kda_fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], init_state=S)
        np.testing.assert_allclose(k[t, 0] @ S[0, 0], v[t, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 4: linear attention
def test_alpha_one_orthonormal_keys_is_linear_attention():
    """alpha=1 and mutually orthonormal keys: the erase term vanishes and KDA is causal
    linear attention with an inclusive mask, O = tril(Q K^T) diag(beta) V."""
    rng = np.random.default_rng(4)
    K, V, T = 16, 7, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm[:T].astype(np.float32).astype(np.float64)  # rows orthonormal (to fp32 rounding)
    q = rng.standard_normal((T, K))
    v = rng.standard_normal((T, V))
    beta = rng.uniform(0, 1, T)
    g = np.zeros((T, K))
    o, _ = oracle.kda_fwd(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None])
    q32 = q.astype(np.float32).astype(np.float64)
    v32 = v.astype(np.float32).astype(np.float64)
    b32 = beta.astype(np.float32).astype(np.float64)
    ref = np.tril(q32 @ k.T) @ (b32[:, None] * v32)
    np.testing.assert_allclose(o[:, 0], ref, rtol=1e-6, atol=1e-6)  # keys orthonormal to ~1e-7


# ---------------------------------------------------------------- pin 5: basis keys
def test_basis_keys_are_per_channel_gated_attention():
    rng = np.random.default_rng(5)
    K, V, T = 10, 3, 8
    perm = rng.permutation(K)[:T]
    k = np.zeros((T, K))
    k[np.arange(T), perm] = 1.0
    q = rng.standard_normal((T, K)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((T, V)).astype(np.float32).astype(np.float64)
    g = np.log(rng.uniform(0.3, 1.0, (T, K))).astype(np.float32).astype(np.float64)
    beta = rng.uniform(0, 1, T).astype(np.float32).astype(np.float64)
    o, _ = oracle.kda_fwd(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None])
    b = np.cumsum(g, axis=0)
    for t in range(T):
        ref = sum(q[t, perm[j]] * np.exp(b[t, perm[j]] - b[j, perm[j]]) * beta[j] * v[j]
                  for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- pin 6: first order in beta
def test_first_order_in_beta_is_diagonal_decay_attention():
    """beta -> eps*beta: to first order the erase term drops and KDA is the diagonal-decay
    family of the Technical Breakdown 3.2, o_t/eps -> sum_j ((q_t*e^{b_t-b_j}).k_j) beta_j v_j."""
    rng = np.random.default_rng(6)
    T, K, V = 10, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, 1, K, V, alpha_lo=0.4)
    eps = 1e-6
    o, _ = oracle.kda_fwd(q, k, v, g, eps * beta)
    b = np.cumsum(g[:, 0], axis=0)
    for t in range(T):
        ref = sum(((q[t, 0] * np.exp(b[t] - b[j])) @ k[j, 0]) * beta[j, 0] * v[j, 0]
                  for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0] / eps, ref, rtol=0, atol=1e-4)


# ---------------------------------------------------------------- pin 7: scalar gate
def test_scalar_gate_is_gated_delta_rule():
    """All channels sharing one alpha_t gives the gated delta rule of the Technical
    Breakdown 3.2, S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T (the pages' 'v k^T'
    transposed to the K x V orientation)."""
    rng = np.random.default_rng(7)
    T, K, V = 15, 5, 6
    q, k, v, _, beta = _rand_inputs(rng, T, 1, K, V)
    a = rng.uniform(0.3, 1.0, T)
    g = np.repeat(np.log(a)[:, None], K, axis=1).astype(np.float32).astype(np.float64)
    a32 = np.exp(g[:, 0])
    o, fin = oracle.kda_fwd(q, k, v, g[:, None, :], beta)
    S = np.zeros((K, V))
    for t in range(T):
        kt = k[t, 0]
        S = a32[t] * ((np.eye(K) - beta[t, 0] * np.outer(kt, kt)) @ S) + beta[t, 0] * np.outer(kt, v[t, 0])
        np.testing.assert_allclose(o[t, 0], S.T @ q[t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- pin 8: stability
def test_zero_values_never_grow_the_state():
    """v=0, unit k, beta in [0,2], alpha<=1: each step is a decay followed by an erase
    (I - beta k k^T) with spectral norm <= 1, so ||S_t||_F cannot increase."""
    rng = np.random.default_rng(8)
    T, K, V = 30, 8, 5
    q, k, _, g, _ = _rand_inputs(rng, T, 1, K, V, alpha_lo=0.7)
    v = np.zeros((T, 1, V))
    beta = rng.uniform(0, 2, (T, 1))
    S = rng.standard_normal((1, 1, K, V))
    prev = np.linalg.norm(S)
    for t in range(T):
        _, S = oracle.kda_fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], init_state=S)
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


# ---------------------------------------------------------------- pin 9: linearity, V permutation
def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(9)
    T, K, V = 13, 5, 4
    q, k, v1, g, beta = _rand_inputs(rng, T, 2, K, V)
    # values on a 2^-10 grid so that v1 + c*v2 is exact in float32, as the oracle sees it
    v1 = np.round(v1 * 1024) / 1024
    v2 = np.round(rng.standard_normal((T, 2, V)) * 1024) / 1024
    S1 = rng.standard_normal((1, 2, K, V))
    S2 = rng.standard_normal((1, 2, K, V))
    c = 0.5  # exact in float32
    oa, fa = oracle.kda_fwd(q, k, v1 + c * v2, g, beta, init_state=S1 + c * S2)
    o1, f1 = oracle.kda_fwd(q, k, v1, g, beta, init_state=S1)
    o2, f2 = oracle.kda_fwd(q, k, v2, g, beta, init_state=S2)
    np.testing.assert_allclose(oa, o1 + c * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fa, f1 + c * f2, rtol=1e-11, atol=1e-11)
    perm = rng.permutation(V)
    op, fp = oracle.kda_fwd(q, k, v1[:, :, perm], g, beta, init_state=S1[..., perm])
    np.testing.assert_allclose(op, o1[:, :, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(fp, f1[..., perm], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- pin 10: state hand-off
def test_split_resume_varlen_and_decode_agree():
    rng = np.random.default_rng(10)
    K, V, H = 6, 5, 3
    lens = [7, 0, 12, 1]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V)
    S0 = rng.standard_normal((len(lens), H, K, V))
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=cu, init_state=S0)
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        # packed == separate
        on, fn = oracle.kda_fwd(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], init_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], on)
        np.testing.assert_array_equal(fin[n], fn[0])
        if L == 0:
            np.testing.assert_array_equal(fin[n], S0[n])  # empty sequence: final = init
            continue
        # split at t and resume from the handed-off state
        t = L // 2
        oa, fa = oracle.kda_fwd(q[s:s + t], k[s:s + t], v[s:s + t], g[s:s + t], beta[s:s + t], init_state=S0[n:n + 1]) if t else (np.zeros((0, H, V)), S0[n:n + 1])
        ob, fb = oracle.kda_fwd(q[s + t:e], k[s + t:e], v[s + t:e], g[s + t:e], beta[s + t:e], init_state=fa)
        np.testing.assert_allclose(np.concatenate([oa, ob]), on, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(fb, fn, rtol=1e-13, atol=1e-13)
        # L decode steps == forward
        st = np.ascontiguousarray(S0[n:n + 1].copy())
        for i in range(L):
            od = oracle.kda_step(q[s + i:s + i + 1], k[s + i:s + i + 1], v[s + i:s + i + 1], g[s + i:s + i + 1], beta[s + i:s + i + 1], st)
            np.testing.assert_allclose(od[0], on[i], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(st, fn, rtol=1e-13, atol=1e-13)


def test_no_leak_across_sequences():
    """Changing one sequence's inputs changes nothing in the others."""
    rng = np.random.default_rng(11)
    K, V, H = 4, 4, 2
    lens = [5, 6, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _rand_inputs(rng, sum(lens), H, K, V)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=cu)
    v2 = v.copy()
    v2[cu[1]:cu[2]] += 1.0
    o2, fin2 = oracle.kda_fwd(q, k, v2, g, beta, cu_seqlens=cu)
    np.testing.assert_array_equal(o[:cu[1]], o2[:cu[1]])
    np.testing.assert_array_equal(o[cu[2]:], o2[cu[2]:])
    assert not np.allclose(o[cu[1]:cu[2]], o2[cu[1]:cu[2]])
    np.testing.assert_array_equal(fin[[0, 2]], fin2[[0, 2]])


def test_head_subset_matches_full():
    rng = np.random.default_rng(12)
    q, k, v, g, beta = _rand_inputs(rng, 9, 4, 5, 3)
    o, fin = oracle.kda_fwd(q, k, v, g, beta)
    os_, fs = oracle.kda_fwd(q, k, v, g, beta, heads=[3, 1])
    np.testing.assert_array_equal(os_, o[:, [3, 1]])
    np.testing.assert_array_equal(fs, fin[:, [3, 1]])


# ---------------------------------------------------------------- input options
# The prologue the option bits select: the gated delta rule's scalar gate ("A Technical
# Breakdown" 3.2), alpha = sigmoid(z) ("Kimi Linear" explainer, Step 2), beta = sigmoid(x) and
# unit-norm q, k (readings). Pinned by textbook values and identities of the activations and by
# closed forms of the recurrence reached through the option path.
def test_log_sigmoid_values():
    ls = oracle.log_sigmoid
    assert ls(0.0) == pytest.approx(-np.log(2.0), rel=0, abs=1e-15)
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(ls(z) - ls(-z), z, rtol=0, atol=1e-12)  # log(s(z)/s(-z)) = z
    assert np.all(np.diff(ls(z)) > 0) and np.all(ls(z) < 0)
    assert ls(40.0) == pytest.approx(-np.exp(-40.0), rel=1e-12)
    assert ls(-800.0) == pytest.approx(-800.0, rel=1e-15)  # no overflow
    np.testing.assert_allclose(ls(np.log(3.0)), np.log(0.75), rtol=1e-15)


def test_sigmoid_values():
    s = oracle.sigmoid
    assert s(0.0) == 0.5
    x = np.linspace(-20, 20, 81)
    np.testing.assert_allclose(s(x) + s(-x), 1.0, rtol=0, atol=1e-15)
    assert s(np.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    assert s(-800.0) == 0.0 and s(800.0) == 1.0


def test_l2_normalize_values():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.1, 10.0, (7, 3, 1))
    y = oracle.l2_normalize(x)
    n2 = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), n2 / (n2 + oracle.L2NORM_EPS), rtol=1e-13)
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1) / np.linalg.norm(y, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)
    assert np.all(oracle.l2_normalize(np.zeros((2, 5))) == 0.0)


def test_scalar_gate_option_is_gated_delta_rule():
    """OPT_SCALAR_GATE with gate logits: S_t = a_t (I - beta k k^T) S_{t-1} + beta k v^T with
    a_t = 1 / (1 + e^{-z_t}), written out per token."""
    rng = np.random.default_rng(8)
    T, H, K, V = 13, 2, 5, 4
    q, k, v, _, beta = _rand_inputs(rng, T, H, K, V)
    z = rng.uniform(-1.0, 4.0, (T, H))
    S0 = rng.standard_normal((1, H, K, V))
    opts = oracle.OPT_SCALAR_GATE | oracle.OPT_GATE_LOGITS
    o, fin = oracle.kda_fwd(q, k, v, z, beta, init_state=S0, options=opts)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            a = 1.0 / (1.0 + np.exp(-z[t, h]))
            kt = k[t, h]
            S = a * ((np.eye(K) - beta[t, h] * np.outer(kt, kt)) @ S) + beta[t, h] * np.outer(kt, v[t, h])
            np.testing.assert_allclose(o[t, h], S.T @ q[t, h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], S, rtol=1e-11, atol=1e-12)


def test_gate_logits_with_tiny_beta_is_pure_decay():
    """OPT_GATE_LOGITS | OPT_BETA_LOGITS, beta logits -60 (beta ~ 1e-26): nothing is written,
    so S_t = Diag(prod_s sigmoid(z_s)) S_0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(9)
    T, K, V = 9, 6, 3
    q = rng.standard_normal((T, 1, K))
    k = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    z = rng.uniform(-2.0, 5.0, (T, 1, K))
    x = np.full((T, 1), -60.0)
    S0 = rng.standard_normal((1, 1, K, V))
    opts = oracle.OPT_GATE_LOGITS | oracle.OPT_BETA_LOGITS
    o, fin = oracle.kda_fwd(q, k, v, z, x, init_state=S0, options=opts)
    dec = np.cumprod(1.0 / (1.0 + np.exp(-z[:, 0, :])), axis=0)  # [T, K]
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], (dec[t][:, None] * S0[0, 0]).T @ q[t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], dec[-1][:, None] * S0[0, 0], rtol=1e-12, atol=1e-12)


def test_l2norm_and_saturated_beta_recall_values():
    """OPT_L2NORM_QK | OPT_BETA_LOGITS with beta logits +40 (beta = 1 in fp64): the keys are
    unit vectors up to the 1e-6 in the norm, so each token's write is recalled exactly along
    its own key, k_t^T S_t = v_t^T, whatever the decay ("A Technical Breakdown" 3.1: the old
    content along k is erased before v is written)."""
    rng = np.random.default_rng(10)
    T, K, V = 11, 8, 5
    q = rng.standard_normal((T, 1, K))
    k = rng.standard_normal((T, 1, K)) * rng.uniform(0.5, 20.0, (T, 1, 1))
    v = rng.standard_normal((T, 1, V))
    g = np.log(rng.uniform(0.3, 1.0, (T, 1, K)))
    x = np.full((T, 1), 40.0)
    opts = oracle.OPT_L2NORM_QK | oracle.OPT_BETA_LOGITS
    for t_end in (4, T):
        _, fin = oracle.kda_fwd(q[:t_end], k[:t_end], v[:t_end], g[:t_end], x[:t_end], options=opts)
        kt = k[t_end - 1, 0] / np.linalg.norm(k[t_end - 1, 0])
        np.testing.assert_allclose(kt @ fin[0, 0], v[t_end - 1, 0], rtol=0, atol=1e-7)


def test_l2norm_option_is_scale_invariant_and_matches_numpy_norm():
    """Scaling raw q and k by positive factors changes nothing beyond the 1e-6 in the norm, and
    the result equals the plain recurrence on q / |q|, k / |k| (numpy's norm) to that level."""
    rng = np.random.default_rng(11)
    T, H, K, V = 10, 2, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, unit_k=False)
    o1, f1 = oracle.kda_fwd(q, k, v, g, beta, options=oracle.OPT_L2NORM_QK)
    c = rng.uniform(2.0, 9.0, (T, H, 1))
    o2, f2 = oracle.kda_fwd(q * c, k / c, v, g, beta, options=oracle.OPT_L2NORM_QK)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5 * np.abs(o1).max())
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, f3 = oracle.kda_fwd(qn, kn, v, g, beta)
    np.testing.assert_allclose(o1, o3, rtol=0, atol=1e-5 * np.abs(o3).max())
    np.testing.assert_allclose(f1, f3, rtol=0, atol=1e-5 * np.abs(f3).max())


def test_decode_step_options_match_fwd():
    """The decode oracle applies the same prologue: one step per token equals kda_fwd."""
    rng = np.random.default_rng(12)
    T, H, K, V = 6, 3, 4, 5
    q, k, v, _, _ = _rand_inputs(rng, T, H, K, V, unit_k=False)
    z = rng.uniform(-1.0, 3.0, (T, H))
    x = rng.uniform(-3.0, 3.0, (T, H))
    opts = 15
    o, fin = oracle.kda_fwd(q, k, v, z, x, options=opts)
    S = np.zeros((1, H, K, V))
    for t in range(T):
        ot = oracle.kda_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], z[t:t + 1], x[t:t + 1], S, options=opts)
        np.testing.assert_allclose(ot[0], o[t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, fin, rtol=1e-13, atol=1e-13)
