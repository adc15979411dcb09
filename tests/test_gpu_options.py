"""The input options (scalar gate, gate and beta logits, q/k normalisation) and the 256-wide
head dims on the GPU, through the C ABI, against the fp64 oracle running the same prologue."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import oracle
import workloads
from gpu_util import TOL, assert_close, np64, oracle_fwd, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")
SG, GL, BL, L2 = kda.OPT_SCALAR_GATE, kda.OPT_GATE_LOGITS, kda.OPT_BETA_LOGITS, kda.OPT_L2NORM_QK
LENGTHS = [1, 63, 64, 65, 0, 127, 200, 129]


def _cu(lengths):
    return torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("opts,dtype,K,V", [
    (SG, torch.bfloat16, 128, 128),
    (GL, torch.bfloat16, 128, 128),
    (BL | L2, torch.bfloat16, 64, 128),
    (SG | GL, torch.float32, 64, 64),
    (SG | GL | BL | L2, torch.float32, 32, 32),
    (SG | GL | BL | L2, torch.bfloat16, 128, 256),
    (0, torch.bfloat16, 128, 256),
    (0, torch.float32, 64, 256),
    (L2, torch.bfloat16, 32, 256),
])
def test_chunk_options_ragged_varlen(opts, dtype, K, V):
    print("chunk options", opts, dtype, K, V, flush=True)
    H = 3
    T = sum(LENGTHS)
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=dtype, device=DEV, seed=opts * 31 + K + V,
                            num_seqs=len(LENGTHS), init_std=0.1)
    cu = _cu(LENGTHS)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu,
                           options=opts)
    o_ref, f_ref = oracle_fwd(inp, cu=cu, options=opts)
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


@pytest.mark.parametrize("opts,dtype,K,V", [
    (GL, torch.bfloat16, 128, 128),
    (GL, torch.bfloat16, 64, 64),
    (GL | BL | L2, torch.bfloat16, 128, 64),
    (SG | GL, torch.bfloat16, 128, 128),
    (SG | GL, torch.float32, 32, 32),
])
def test_chunk_strong_gate_logits(opts, dtype, K, V):
    """Gate logits z ~ U(-12, -6): alpha = sigmoid(z) between e^{-12} and e^{-6} per token, the
    range trained gates reach; the in-chunk decays over 16 tokens leave fp32 range by far."""
    print("chunk strong gate logits", opts, dtype, K, V, flush=True)
    H = 2
    T = sum(LENGTHS)
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=dtype, device=DEV, seed=opts + K + 3,
                            num_seqs=len(LENGTHS), init_std=0.1, gate_logit_range=(-12.0, -6.0))
    cu = _cu(LENGTHS)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu,
                           options=opts)
    o_ref, f_ref = oracle_fwd(inp, cu=cu, options=opts)
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


def test_chunk_all_options_long_sampled_heads():
    """Every option on the long-prefill shape (T=65536, H=32, K=V=128, bf16): the gated delta
    rule with gate and beta logits and unit-norm q, k; two heads against the oracle."""
    print("chunk all options long", flush=True)
    T, H, K, V = 65536, 32, 128, 128
    opts = SG | GL | BL | L2
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=torch.bfloat16, device=DEV, seed=77,
                            init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], options=opts)
    heads = [2, 29]
    o_ref, f_ref = oracle_fwd(inp, heads=heads, options=opts)
    assert_close(np64(o[:, heads]), o_ref, torch.bfloat16, "o")
    assert_close(np64(fin[:, heads]), f_ref, torch.bfloat16, "final")


def test_chunk_options_match_recurrent():
    """The chunked and the recurrent path agree with every option set."""
    print("chunk vs recurrent with options", flush=True)
    T, H, K, V = 200, 2, 128, 128
    opts = SG | GL | BL | L2
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=torch.bfloat16, device=DEV, seed=5,
                            init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], options=opts)
    st = inp["init_state"].clone()
    od = torch.empty_like(o)
    for t in range(T):
        od[t] = kda.decode_step(*(inp[x][t:t + 1] for x in ORDER), state=st, options=opts)[0]
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(o), np64(od)) <= tol
    assert rel_err(np64(fin), np64(st)) <= tol


@pytest.mark.parametrize("opts,dtype,K,V,N,H", [
    (SG | GL | BL | L2, torch.bfloat16, 256, 256, 2, 2),
    (SG | GL, torch.float32, 128, 256, 2, 3),
    (L2, torch.bfloat16, 256, 64, 3, 2),
    (0, torch.bfloat16, 256, 128, 2, 2),
    (BL, torch.float32, 32, 256, 4, 1),
    (GL | L2, torch.bfloat16, 128, 128, 4, 4),
    (BL | L2, torch.bfloat16, 32, 64, 3, 2),   # unit norm over fewer key channels than lanes
    (SG | L2, torch.float32, 64, 32, 2, 3),
])
def test_decode_options(opts, dtype, K, V, N, H):
    print("decode options", opts, dtype, K, V, N, H, flush=True)
    steps = 3
    gen = torch.Generator(device=DEV)
    gen.manual_seed(opts + K + V)
    state = 0.1 * torch.randn((N, H, K, V), generator=gen, device=DEV)
    ref = np64(state).copy()
    for s in range(steps):
        inp = workloads.gen_raw(N, H, K, V, opts, dtype=dtype, device=DEV, seed=100 * s + opts)
        o = torch.full((N, H, V), float("nan"), dtype=dtype, device=DEV)
        kda.decode_step(*(inp[x] for x in ORDER), state=state, o=o, options=opts)
        o_ref = oracle.kda_step(*(np64(inp[x]) for x in ORDER), ref, options=opts)
        assert_close(np64(o), o_ref, dtype, "o step %d" % s)
        assert_close(np64(state), ref, dtype, "state step %d" % s)
