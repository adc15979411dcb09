"""Helpers shared by the GPU parity tests (comparison against the fp64 oracle)."""
import numpy as np
import torch

import oracle

# max-abs(GPU - oracle) <= TOL * max|oracle|
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    scale = max(float(np.abs(ref).max()), 1e-30)
    return float(np.abs(got - ref).max()) / scale


def oracle_fwd(inp, cu=None, heads=None, options=0):
    """Run the oracle on exactly the tensors the GPU received."""
    cu_np = None if cu is None else cu.cpu().numpy().astype(np.int64)
    init = inp.get("init_state")
    init_np = None if init is None else np64(init)
    return oracle.kda_fwd(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["log_alpha"]),
                          np64(inp["beta"]), cu_seqlens=cu_np, init_state=init_np, heads=heads,
                          options=options)


def assert_close(got, ref, dtype, what):
    err = rel_err(got, ref)
    tol = TOL[dtype]
    assert np.all(np.isfinite(np.asarray(got))), "%s: non-finite values" % what
    assert err <= tol, "%s: max-abs error / max|ref| = %.3e > %.1e" % (what, err, tol)
    return err
