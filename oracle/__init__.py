"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path (the HIP library and its
Python binding) never does, and shares no code with it.

The recurrence lives in ``kda_oracle.c`` (plain C, fp64, one token at a time, OpenMP over
(sequence, head)). This module builds/loads that file, marshals numpy arrays, and applies
the optional input prologue (``apply_options``) in fp64 numpy before the recurrence.
Inputs are converted to float64, which is exact for bf16 and fp32 values, so the oracle
consumes exactly the numbers the GPU received.

The definition it follows is the KDA update of "Kimi Linear's Hybrid Linear Attention
Architecture: A Technical Breakdown" section 3.3 (decay, then erase along k, then write),
with the orientation of the update-rule code block of "Kimi Linear: How Moonshot AI Built
a Hybrid Attention Architecture That Beats Full Attention" (S is K x V, write k v^T), and
the output read after the write ("Kimi Linear" explainer, "Step 4: Query").

Input options (the bit values of the library's public option flags):
  OPT_SCALAR_GATE  one gate value per token and head, shared by every key channel: the gated
                   delta rule of "A Technical Breakdown", section 3.2 (the whole memory decays
                   by one scalar before the erase and write).
  OPT_GATE_LOGITS  the gate input is z with alpha = sigmoid(z) ("Kimi Linear" explainer,
                   "Step 2: Per-Channel Decay"), so log alpha = log sigmoid(z).
  OPT_BETA_LOGITS  the beta input is x with beta = sigmoid(x) (a reading: the pages call beta
                   a learned write strength in (0, 1) without fixing its activation).
  OPT_L2NORM_QK    q and k are scaled to unit L2 norm per token and head (a reading of the
                   L2-normalised q and k of the workloads), x / sqrt(sum x^2 + 1e-6).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_kda_oracle.so")
_lock = threading.Lock()
_lib = None

OPT_SCALAR_GATE = 1
OPT_GATE_LOGITS = 2
OPT_BETA_LOGITS = 4
OPT_L2NORM_QK = 8
L2NORM_EPS = 1e-6


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math) into oracle/_kda_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            f = lib.kda_oracle_fwd
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 4 + [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int32]
            s = lib.kda_oracle_step
            s.restype = ctypes.c_int
            s.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int32] * 4 + [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
            b = lib.kda_oracle_bwd
            b.restype = ctypes.c_int
            b.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 9 + [
                ctypes.c_int32]
            lib.kda_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    """Number of OpenMP threads the oracle uses by default."""
    return int(_load().kda_oracle_max_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def log_sigmoid(z):
    """log(1 / (1 + e^{-z})) in fp64, as -log(e^0 + e^{-z}) through numpy's logaddexp, which
    does not overflow for any finite z."""
    return -np.logaddexp(0.0, -np.asarray(z, dtype=np.float64))


def sigmoid(x):
    """1 / (1 + e^{-x}) in fp64, as exp(log_sigmoid(x))."""
    return np.exp(log_sigmoid(x))


def l2_normalize(x, eps: float = L2NORM_EPS):
    """x / sqrt(sum of squares over the last axis + eps), fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def apply_options(q, k, gate, beta, options: int):
    """The input prologue selected by ``options`` (OPT_* bits), in fp64.

    q, k: [..., K]; gate: [..., K], or [...] with OPT_SCALAR_GATE; beta: [...].
    Returns (q, k, log_alpha [..., K], beta) ready for the recurrence.
    """
    q, k, g, b = _f64(q), _f64(k), _f64(gate), _f64(beta)
    K = q.shape[-1]
    if options & OPT_L2NORM_QK:
        q, k = l2_normalize(q), l2_normalize(k)
    if options & OPT_GATE_LOGITS:
        g = log_sigmoid(g)
    if options & OPT_SCALAR_GATE:
        g = np.repeat(g[..., None], K, axis=-1)
    if options & OPT_BETA_LOGITS:
        b = sigmoid(b)
    return q, k, np.ascontiguousarray(g), b


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def kda_fwd(q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None, heads=None,
            threads: int = 0, options: int = 0):
    """Token-by-token fp64 KDA forward.

    q, k, log_alpha: [T, H, K]; v: [T, H, V]; beta: [T, H] (any float dtype numpy arrays).
    options: OPT_* bits (log_alpha is [T, H] with OPT_SCALAR_GATE); see apply_options.
    cu_seqlens: [N+1] int (None = one sequence of length T).
    init_state: [N, H, K, V] (None = zeros).
    heads: optional list of head indices to compute (outputs then hold only those heads).
    Returns (o [T, Hs, V] float64, final_state [N, Hs, K, V] float64).
    """
    lib = _load()
    q, k, g, b = apply_options(q, k, log_alpha, beta, options)
    v = _f64(v)
    T, H, K = q.shape
    V = v.shape[2]
    assert k.shape == (T, H, K) and g.shape == (T, H, K) and v.shape[:2] == (T, H)
    assert b.shape == (T, H)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    if heads is None:
        hs = None
        nsel = H
    else:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        nsel = hs.shape[0]
    init = None
    if init_state is not None:
        init = np.ascontiguousarray(np.asarray(init_state, dtype=np.float64))
        assert init.shape == (N, H, K, V)
    o = np.zeros((T, nsel, V), dtype=np.float64)
    fin = np.zeros((N, nsel, K, V), dtype=np.float64)
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(cu), N, H, K, V,
                            _ptr(init) if init is not None else None,
                            _ptr(hs) if hs is not None else None, nsel, _ptr(o), _ptr(fin),
                            int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed (%d)" % rc)
    return o, fin


def kda_step(q, k, v, log_alpha, beta, state: np.ndarray, threads: int = 0, options: int = 0):
    """One fp64 recurrent step for N x H heads; ``state`` [N, H, K, V] float64 is updated
    in place. q, k, log_alpha: [N, H, K] (log_alpha [N, H] with OPT_SCALAR_GATE);
    v: [N, H, V]; beta: [N, H]. Returns o [N, H, V]."""
    lib = _load()
    q, k, g, b = apply_options(q, k, log_alpha, beta, options)
    v = _f64(v)
    N, H, K = q.shape
    V = v.shape[2]
    assert state.dtype == np.float64 and state.flags["C_CONTIGUOUS"]
    assert state.shape == (N, H, K, V)
    o = np.zeros((N, H, V), dtype=np.float64)
    rc = lib.kda_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), N, H, K, V,
                             _ptr(state), _ptr(o), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_step failed (%d)" % rc)
    return o


def kda_bwd(q, k, v, log_alpha, beta, dout, dfinal=None, cu_seqlens=None, init_state=None,
            threads: int = 0):
    """Gradients of kda_fwd for the loss sum(dout * o) + sum(dfinal * final_state), fp64.

    Shapes as in kda_fwd; dout [T, H, V], dfinal [N, H, K, V] or None (zero).
    Returns (dq, dk, dv, dlog_alpha, dbeta, dinit_state) as float64 arrays.
    """
    lib = _load()
    q, k, v, g, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    do = _f64(dout)
    T, H, K = q.shape
    V = v.shape[2]
    assert k.shape == (T, H, K) and g.shape == (T, H, K) and v.shape == (T, H, V)
    assert b.shape == (T, H) and do.shape == (T, H, V)
    cu = (np.array([0, T], dtype=np.int64) if cu_seqlens is None else
          np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64)))
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    init = None if init_state is None else _f64(init_state)
    dfin = None if dfinal is None else _f64(dfinal)
    for a in (init, dfin):
        assert a is None or a.shape == (N, H, K, V)
    dq, dk, dg = (np.zeros((T, H, K)) for _ in range(3))
    dv = np.zeros((T, H, V))
    db = np.zeros((T, H))
    dinit = np.zeros((N, H, K, V))
    P = lambda a: None if a is None else _ptr(a)
    rc = lib.kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(cu), N, H, K, V,
                            P(init), _ptr(do), P(dfin), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                            _ptr(db), _ptr(dinit), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed (%d)" % rc)
    return dq, dk, dv, dg, db, dinit


def kda_bwd_options(q, k, v, gate, beta, dout, options: int, dfinal=None, cu_seqlens=None,
                    init_state=None, threads: int = 0):
    """Gradients with respect to the raw inputs of kda_fwd on apply_options(q, k, gate, beta),
    fp64: kda_bwd on the processed inputs, then the chain rule through each option.

    gate is [T, H, K], or [T, H] with OPT_SCALAR_GATE (and so is its gradient). The options'
    derivatives: unit norm y = x r, r = (|x|^2 + eps)^{-1/2}, gives dx = r dy - r^3 x (x . dy);
    log alpha = log sigmoid(z) gives dz = dlog_alpha sigmoid(-z); one gate per head sums the
    channels' gradients; beta = sigmoid(x) gives dx = dbeta sigmoid(x) sigmoid(-x).
    Returns (dq, dk, dv, dgate, dbeta, dinit_state).
    """
    q0, k0, z0, b0 = _f64(q), _f64(k), _f64(gate), _f64(beta)
    qp, kp, gp, bp = apply_options(q0, k0, z0, b0, options)
    dq, dk, dv, dg, db, dinit = kda_bwd(qp, kp, v, gp, bp, dout, dfinal=dfinal,
                                        cu_seqlens=cu_seqlens, init_state=init_state,
                                        threads=threads)
    if options & OPT_L2NORM_QK:
        def back(x, dy):
            r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)
            return r * dy - r ** 3 * x * np.sum(x * dy, axis=-1, keepdims=True)
        dq, dk = back(q0, dq), back(k0, dk)
    if options & OPT_SCALAR_GATE:
        dg = np.sum(dg, axis=-1)
    if options & OPT_GATE_LOGITS:
        dg = dg * sigmoid(-z0)
    if options & OPT_BETA_LOGITS:
        db = db * sigmoid(b0) * sigmoid(-b0)
    return dq, dk, dv, dg, db, dinit
