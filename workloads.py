"""Seeded synthetic inputs for the KDA workloads.

This module holds input generation only (random draws, L2 normalisation of q and k,
casts); none of the operator's arithmetic. Both the HIP path's tests/benchmark and the
oracle consume what it produces.

Workloads (head dim 128 and 32 heads up to 1M tokens stand in for the long-context use
the pages describe; the pages print no dataset the operator is measured on):

  tiny     N=1, H=1, T=256, K=V=32, fp32, numpy default_rng(0), draw order q,k,v,alpha,beta,
           q and k L2-normalised per token, alpha ~ U[0.9,1) passed as log alpha,
           beta ~ U(0,1), zero initial state.
  med      N=2 equal sequences of 4096, H=8, K=V=128, bf16; log alpha = -softplus(z)*0.1,
           beta = sigmoid(z'), zero initial state.
  long     N=1, H=32, T=65536, K=V=128, bf16, gates as in 'tiny', init state 0.1*N(0,1).
  varlen   16 sequences (lengths below, total 129,148), H=32, K=V=128, bf16, gates as in
           'tiny', per-sequence init states 0.1*N(0,1).
  decode   N=256 sequences, H=32, K=V=128, fp32 state 0.1*N(0,1), bf16 step inputs drawn
           as in 'tiny'; and a 1,048,576-token single-sequence prefill with zero init.
"""
from __future__ import annotations

import math

import numpy as np

VARLEN_LENGTHS = [19154, 1788, 7076, 3667, 2156, 3899, 4515, 8520, 13142, 1079, 2469, 8310,
                  1368, 32515, 18327, 1163]


def varlen_lengths_rule(n: int = 16, lo: int = 1024, hi: int = 32768, target: int = 131072,
                        rel: float = 0.05):
    """First seed s >= 0 of numpy default_rng(s) whose n log-uniform draws on [lo, hi]
    (floor of exp of a uniform draw in log space) total within +-rel of target."""
    for s in range(10000):
        rng = np.random.default_rng(s)
        x = rng.uniform(math.log(lo), math.log(hi), n)
        lens = np.floor(np.exp(x)).astype(np.int64)
        if abs(int(lens.sum()) - target) <= rel * target:
            return s, [int(v) for v in lens]
    raise RuntimeError("no seed found")


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _l2n_np(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def tiny_numpy(T: int = 256, H: int = 1, K: int = 32, V: int = 32, seed: int = 0):
    """The fp32 'tiny' workload as float32 numpy arrays (draw order q,k,v,alpha,beta)."""
    rng = np.random.default_rng(seed)
    q = _l2n_np(rng.standard_normal((T, H, K))).astype(np.float32)
    k = _l2n_np(rng.standard_normal((T, H, K))).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    alpha = rng.uniform(0.9, 1.0, (T, H, K))
    beta = rng.uniform(0.0, 1.0, (T, H)).astype(np.float32)
    log_alpha = np.log(alpha).astype(np.float32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta)


# ---------------------------------------------------------------- torch generators
def _torch():
    import torch
    return torch


def gen_forward(T_total: int, H: int, K: int, V: int, *, gates: str = "uniform",
                dtype=None, device="cpu", seed: int = 0, num_seqs: int = 1,
                init_std: float | None = None, block_tokens: int = 65536):
    """Seeded torch inputs for kda_chunk_fwd, laid out token-major [T, H, .].

    gates: 'uniform' (alpha ~ U[0.9,1), beta ~ U(0,1)), 'slow' (alpha ~ U[0.999,1), beta ~
    U(0,1): the state keeps a visible share of its past over a few hundred tokens) or
    'softplus' (log alpha = -softplus(z)*0.1, beta = sigmoid(z')). q, k are drawn N(0,1) and
    L2-normalised per token and head in fp32, then every tensor is cast to ``dtype``.
    Generated in token blocks to bound peak memory; init_state (fp32) only if init_std.
    """
    torch = _torch()
    dtype = dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name, last in (("q", K), ("k", K), ("v", V), ("log_alpha", K), ("beta", None)):
        shape_tail = (H, last) if last is not None else (H,)
        t = torch.empty((T_total,) + shape_tail, dtype=dtype, device=device)
        for s in range(0, T_total, block_tokens):
            e = min(T_total, s + block_tokens)
            shp = (e - s,) + shape_tail
            if name in ("q", "k"):
                x = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
                x = x / x.norm(dim=-1, keepdim=True)
            elif name == "v":
                x = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
            elif name == "log_alpha":
                if gates in ("uniform", "slow"):
                    lo = 0.9 if gates == "uniform" else 0.999
                    x = torch.log(lo + (1.0 - lo) * torch.rand(shp, generator=gen, device=device,
                                                               dtype=torch.float32))
                else:
                    z = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
                    x = -torch.nn.functional.softplus(z) * 0.1
            else:
                if gates in ("uniform", "slow"):
                    x = torch.rand(shp, generator=gen, device=device, dtype=torch.float32)
                else:
                    z = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
                    x = torch.sigmoid(z)
            t[s:e] = x.to(dtype)
        out[name] = t
    if init_std is not None:
        out["init_state"] = init_std * torch.randn((num_seqs, H, K, V), generator=gen,
                                                   device=device, dtype=torch.float32)
    else:
        out["init_state"] = None
    return out


# option bits of the operator's input prologue (the public KDA_OPT_* values)
OPT_SCALAR_GATE, OPT_GATE_LOGITS, OPT_BETA_LOGITS, OPT_L2NORM_QK = 1, 2, 4, 8


def gen_raw(T_total: int, H: int, K: int, V: int, options: int, *, dtype=None, device="cpu",
            seed: int = 0, num_seqs: int = 1, init_std: float | None = None,
            gate_logit_range=(2.0, 7.0)):
    """Seeded raw inputs for the option bits, token-major:
    q, k ~ N(0,1), times U(0.5, 4) per token and head with OPT_L2NORM_QK (left for the kernel
    to normalise), else L2-normalised here; v ~ N(0,1); the gate [T, H, K] or, with
    OPT_SCALAR_GATE, [T, H]: logits z ~ U(gate_logit_range), by default U(2, 7), with
    OPT_GATE_LOGITS (alpha = sigmoid(z) in [0.88, 0.999]; U(-12, -6) gives the strong decays
    alpha ~ e^{-6} .. e^{-12}), else log alpha = log U[0.9, 1); beta logits ~ 1.5 N(0,1) with
    OPT_BETA_LOGITS, else beta ~ U(0, 1). Every tensor is cast to ``dtype``."""
    torch = _torch()
    dtype = dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    f = dict(generator=gen, device=device, dtype=torch.float32)
    out = {}
    for name in ("q", "k"):
        x = torch.randn((T_total, H, K), **f)
        if options & OPT_L2NORM_QK:
            x = x * (0.5 + 3.5 * torch.rand((T_total, H, 1), **f))
        else:
            x = x / x.norm(dim=-1, keepdim=True)
        out[name] = x.to(dtype)
    out["v"] = torch.randn((T_total, H, V), **f).to(dtype)
    gshape = (T_total, H) if options & OPT_SCALAR_GATE else (T_total, H, K)
    if options & OPT_GATE_LOGITS:
        lo, hi = gate_logit_range
        g = lo + (hi - lo) * torch.rand(gshape, **f)
    else:
        g = torch.log(0.9 + 0.1 * torch.rand(gshape, **f))
    out["log_alpha"] = g.to(dtype)
    if options & OPT_BETA_LOGITS:
        b = 1.5 * torch.randn((T_total, H), **f)
    else:
        b = torch.rand((T_total, H), **f)
    out["beta"] = b.to(dtype)
    out["init_state"] = (None if init_std is None else
                         init_std * torch.randn((num_seqs, H, K, V), **f))
    return out


def gen_decode_inputs(N: int, H: int, K: int, V: int, *, dtype=None, device="cpu",
                      gen=None, seed: int = 0):
    """One decode step's inputs [N, H, .] drawn as in the 'tiny' workload."""
    torch = _torch()
    dtype = dtype or torch.bfloat16
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
    q = torch.randn((N, H, K), generator=gen, device=device)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = torch.randn((N, H, K), generator=gen, device=device)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn((N, H, V), generator=gen, device=device).to(dtype)
    g = torch.log(0.9 + 0.1 * torch.rand((N, H, K), generator=gen, device=device)).to(dtype)
    b = torch.rand((N, H), generator=gen, device=device).to(dtype)
    return dict(q=q, k=k, v=v, log_alpha=g, beta=b)


WORKLOADS = {
    "tiny": dict(num_seqs=1, H=1, T=256, K=32, V=32, dtype="float32", gates="uniform",
                 init_std=None, seed=0),
    "med": dict(num_seqs=2, H=8, T=4096, K=128, V=128, dtype="bfloat16", gates="softplus",
                init_std=None, seed=2),
    "long": dict(num_seqs=1, H=32, T=65536, K=128, V=128, dtype="bfloat16", gates="uniform",
                 init_std=0.1, seed=3),
    "varlen": dict(num_seqs=16, H=32, T=None, K=128, V=128, dtype="bfloat16", gates="uniform",
                   init_std=0.1, seed=4, lengths=VARLEN_LENGTHS),
    "prefill1m": dict(num_seqs=1, H=32, T=1048576, K=128, V=128, dtype="bfloat16",
                      gates="uniform", init_std=None, seed=5),
    "decode": dict(num_seqs=256, H=32, K=128, V=128, dtype="bfloat16", steps=512,
                   state_std=0.1, seed=5),
}


def make_workload(name: str, device="cpu"):
    """Inputs of a named forward workload as torch tensors on ``device`` plus cu_seqlens
    (int32 torch tensor, or None for equal-length sequences)."""
    torch = _torch()
    w = WORKLOADS[name]
    dtype = getattr(torch, w["dtype"])
    if name == "tiny":
        d = tiny_numpy(T=w["T"], H=w["H"], K=w["K"], V=w["V"], seed=w["seed"])
        out = {kk: torch.from_numpy(vv).to(device) for kk, vv in d.items()}
        out["init_state"] = None
        out["cu_seqlens"] = None
        out["num_seqs"] = 1
        return out
    if "lengths" in w:
        cu = cu_from_lengths(w["lengths"])
        T_total = int(cu[-1])
    else:
        T_total = w["T"] * w["num_seqs"]
        cu = None
    out = gen_forward(T_total, w["H"], w["K"], w["V"], gates=w["gates"], dtype=dtype,
                      device=device, seed=w["seed"], num_seqs=w["num_seqs"],
                      init_std=w["init_std"])
    out["cu_seqlens"] = None if cu is None else torch.from_numpy(cu.astype(np.int32)).to(device)
    out["num_seqs"] = w["num_seqs"]
    return out
